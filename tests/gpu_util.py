"""Helpers for the GPU parity tests: run the HIP layer through the C ABI and compare it with the
CPU oracle on the same seeded inputs."""
from __future__ import annotations

import os
import sys
import time

import numpy as np
import torch

import oracle
import synth

RTOL_L2 = 5e-3        # FFN outputs: relative L2 error against the fp32 oracle
RTOL_MAXABS = 3e-2    # FFN outputs: max abs error / max |ref|
WTOL = 1e-6           # routing weights: absolute
WORKERS = min(16, os.cpu_count() or 1)


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def device_bank(canon: synth.Bank):
    import routed_expert_ffn_wave_amd as ft
    c = canon.to("cuda")
    return ft.ft_moe_pack_bank(c.fmt, c.n_slots, c.d, c.I, c.w13, c.w2, c.s13, c.s2)


def ffn_errors(got: np.ndarray, ref: np.ndarray):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    nref = np.linalg.norm(ref)
    mref = np.abs(ref).max() if ref.size else 0.0
    rel = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got)
    mx = np.abs(got - ref).max() / mref if mref > 0 else (np.abs(got).max() if got.size else 0.0)
    return rel, mx


def assert_ffn_close(got, ref, what: str):
    rel, mx = ffn_errors(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert rel <= RTOL_L2 and mx <= RTOL_MAXABS, f"{what}: rel-L2 {rel:.3e} (<= {RTOL_L2}), max-abs/max {mx:.3e}"
    return rel, mx


def run_gpu_layer(li: synth.LayerInputs, bank_dev, flags=0, mode="layer"):
    """Run the layer through MoELayer: one ft_moe_layer call ("layer", the benchmark's launch
    configuration) or the four separate calls ("calls")."""
    import routed_expert_ffn_wave_amd as ft
    w = li.workload
    T = li.T
    layer = ft.MoELayer(bank_dev, li.slot_of_expert.cuda(), w.k, T, shared_slot=w.shared_slot, flags=flags, mode=mode)
    logits = li.logits.cuda()
    x = li.x.cuda()
    out, mask = layer.forward(logits, x)
    torch.cuda.synchronize()
    assert layer.status_word() == 0, "a dependency wait of the fused kernel gave up"
    n = T * w.k
    return dict(ids=layer.ids[:T].cpu().numpy(), w=layer.w[:T].cpu().numpy(), counts=layer.counts.cpu().numpy(),
                offsets=layer.offsets.cpu().numpy(), gather=layer.gather[:n].cpu().numpy(),
                inv=layer.inv[:n].cpu().numpy(), y_sorted=layer.y_sorted[:n],
                y_shared=None if layer.y_shared is None else layer.y_shared[:T],
                out=out.float().cpu().numpy(), mask=mask.cpu().numpy().astype(np.uint32))


def compare_layer(li: synth.LayerInputs, g: dict, tokens=None, label=""):
    """Oracle on the same inputs (all tokens, or a sample); bit-exact routing/permutation/mask,
    FFN and output within the stated tolerance.  Returns the oracle dict and error figures."""
    w = li.workload
    t0 = time.time()
    ora = oracle.layer(li.logits, li.x, li.bank, li.slot_of_expert, w.k, shared_slot=w.shared_slot, tokens=tokens,
                       workers=WORKERS)
    t_ora = time.time() - t0
    assert np.array_equal(g["ids"], ora["ids"]), f"{label}: ids differ"
    assert np.abs(g["w"] - ora["w"]).max() <= WTOL, f"{label}: weights differ by {np.abs(g['w'] - ora['w']).max()}"
    assert np.array_equal(g["counts"], ora["counts"]), f"{label}: counts differ"
    assert np.array_equal(g["offsets"], ora["offsets"]), f"{label}: offsets differ"
    assert np.array_equal(g["gather"], ora["gather"]), f"{label}: gather differs"
    assert np.array_equal(g["inv"], ora["inv"]), f"{label}: inv differs"
    tok = ora["tokens"]
    assert np.array_equal(g["mask"][tok], ora["mask"][tok]), f"{label}: residual mask differs"
    errs = {}
    if len(ora["y_pos"]):
        ys = g["y_sorted"][torch.from_numpy(ora["y_pos"]).cuda()].float().cpu().numpy()
        errs["y"] = assert_ffn_close(ys, ora["y_rows"], f"{label} y_sorted")
    if ora["y_shared"] is not None:
        errs["y_shared"] = assert_ffn_close(g["y_shared"].float().cpu().numpy()[tok], ora["y_shared"][tok],
                                            f"{label} y_shared")
    errs["out"] = assert_ffn_close(g["out"][tok], ora["out"][tok], f"{label} out")
    log(f"{label}: ok; oracle {t_ora:.1f}s on {len(tok)} tokens; errors " +
        ", ".join(f"{k} rel-L2 {v[0]:.2e} max {v[1]:.2e}" for k, v in errs.items()))
    return ora, errs


def run_gpu_layer_graph(li: synth.LayerInputs, bank_dev, replays: int = 2):
    """The benchmark's launch configuration: MoELayer's four calls captured once into a HIP graph
    on a side stream and replayed; every replay must reproduce the eager result bit for bit.
    `li` may hold device tensors (inputs generated on the GPU)."""
    import routed_expert_ffn_wave_amd as ft
    w = li.workload
    T = li.T
    layer = ft.MoELayer(bank_dev, li.slot_of_expert.cuda(), w.k, T, shared_slot=w.shared_slot)
    logits, x = li.logits.cuda(), li.x.cuda()
    out, mask = layer.forward(logits, x)
    eager = out.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        layer.forward(logits, x)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            layer.forward(logits, x)
    torch.cuda.synchronize()
    for _ in range(replays):
        layer.out.zero_()
        layer.y_sorted.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out[:T], eager), "graph replay differs from the eager layer"
        assert layer.status_word() == 0, "a dependency wait of the fused kernel gave up"
    n = T * w.k
    return dict(ids=layer.ids[:T].cpu().numpy(), w=layer.w[:T].cpu().numpy(), counts=layer.counts.cpu().numpy(),
                offsets=layer.offsets.cpu().numpy(), gather=layer.gather[:n].cpu().numpy(),
                inv=layer.inv[:n].cpu().numpy(), y_sorted=layer.y_sorted[:n],
                y_shared=None if layer.y_shared is None else layer.y_shared[:T],
                out=layer.out[:T].float().cpu().numpy(), mask=layer.mask[:T].cpu().numpy().astype(np.uint32))


def host_inputs(li: synth.LayerInputs) -> synth.LayerInputs:
    """Host copy of device-generated inputs, for the oracle."""
    return synth.LayerInputs(li.workload, li.layer, li.T, li.logits.cpu(), li.x.cpu(), li.slot_of_expert.cpu(),
                             li.bank.to("cpu"))


def sample_tokens(T: int, n: int, seed: int):
    """A seeded sample of n tokens that always holds the first and the last token."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], mid]))
