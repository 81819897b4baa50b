"""GPU parity at the workloads' full sizes, in the benchmark's launch configuration: MoELayer's four
calls captured into a HIP graph and replayed.  Inputs follow the seeded recipe, generated on the GPU
(large banks) and copied to the host for the oracle.  Routing, permutation and mask are compared
bit for bit over the whole layer; FFN rows and outputs over every token where the oracle finishes
in seconds (the bf16 prefill layer of 4096 tokens included), else over a seeded token sample that
holds the first and last token and, for the Zipf-routed resident bank, every token of the smallest
expert groups."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import compare_layer, device_bank, host_inputs, log, run_gpu_layer_graph, sample_tokens

pytestmark = pytest.mark.gpu
W = synth.WORKLOADS


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_expert_ffn_wave_amd as ft
    return ft


def _inputs(w: synth.Workload, layer: int, T: int, bank=None):
    """Device inputs of one layer; `bank` reuses an already generated (canonical, host) bank."""
    L = synth.logits(w, layer, T, device="cuda")
    x = synth.activations(w, layer, T, device="cuda")
    slot = synth.slot_table(w, layer)
    if bank is None:
        bank = synth.make_bank(w, layer, device="cuda").to("cpu")
    return synth.LayerInputs(w, layer, T, L, x, slot, bank)


def _make_bank(w: synth.Workload, layer: int):
    """synth.make_bank on the GPU, slot by slot with progress lines."""
    experts = synth.slot_experts(w, layer)
    bank = synth.empty_bank(w.fmt, len(experts), w.d, w.I, device="cuda")
    for s, e in enumerate(experts):
        w13, w2 = synth.expert_weights(w, layer, e, device="cuda")
        synth.fill_slot(bank, s, w13, w2)
        if (s + 1) % 32 == 0 or s + 1 == len(experts):
            torch.cuda.synchronize()
            log(f"{w.name}: {s + 1}/{len(experts)} slots generated")
    return bank


def _small_group_tokens(host, n_groups: int):
    """Every token of the n_groups smallest non-empty resident expert groups (their rows sit in the
    partly filled tail tiles of the GEMM kernels), from the oracle's routing of the same logits."""
    w = host.workload
    ids, _ = oracle.route(host.logits, w.k)
    slot = host.slot_of_expert.numpy()
    counts = np.bincount(ids.reshape(-1), minlength=w.E)
    groups = [e for e in np.argsort(counts, kind="stable") if counts[e] > 0 and slot[e] >= 0][:n_groups]
    return np.unique(np.nonzero(np.isin(ids, groups).any(axis=1))[0])


def _check(ft, li, bank_dev, n_sample: int, label: str, small_groups: int = 0):
    log(f"{label}: T={li.T} d={li.workload.d} E={li.workload.E} k={li.workload.k} I={li.workload.I}")
    g = run_gpu_layer_graph(li, bank_dev)
    host = host_inputs(li)
    tokens = None if li.T <= n_sample else sample_tokens(li.T, n_sample, seed=li.T + 17 * li.layer)
    if tokens is not None and small_groups:
        tokens = np.union1d(tokens, _small_group_tokens(host, small_groups))
    compare_layer(host, g, tokens=tokens, label=label)


@pytest.mark.parametrize("layer", [0, 47])
def test_decode_q4_0_full(ft, layer):
    w = W["decode_q4_0"]
    li = _inputs(w, layer, w.T)
    _check(ft, li, device_bank(li.bank), n_sample=w.T, label=f"decode_q4_0 layer {layer}")


@pytest.mark.parametrize("T", [10, 12])
def test_decode_q4_0_batch_sizes(ft, T):
    """The decode shape at batch sizes between the 8-token workload and the one-launch path's
    limit (two segments of 64 routed pairs in its bookkeeping, 1400-1700 gate/up items, more than
    the blocks resident at once); every token against the oracle."""
    w = W["decode_q4_0"].replace(T=T)  # the recipe's tensors drawn for T tokens
    li = _inputs(w, 3, T)
    _check(ft, li, device_bank(li.bank), n_sample=T, label=f"decode_q4_0 T={T}")


def test_prefill_bf16_zipf_full(ft):
    w = W["prefill_bf16_zipf"]
    li = _inputs(w, 0, w.T)
    _check(ft, li, device_bank(li.bank), n_sample=w.T, label="prefill_bf16_zipf")  # every token


@pytest.fixture(scope="module")
def mxfp4_bank(ft):
    w = W["mxfp4_shared"]
    log("generating the mxfp4_shared bank (257 slots)")
    canon = _make_bank(w, 0)
    host = canon.to("cpu")
    dev = device_bank(canon)
    del canon
    torch.cuda.empty_cache()
    return host, dev


@pytest.mark.parametrize("T,n_sample", [(16, 16), (8192, 8)])
def test_mxfp4_shared_full(ft, mxfp4_bank, T, n_sample):
    w = W["mxfp4_shared"]
    host, dev = mxfp4_bank
    li = _inputs(w, 0, T, bank=host)
    _check(ft, li, dev, n_sample=n_sample, label=f"mxfp4_shared T={T}")


@pytest.fixture(scope="module")
def fp8_bank(ft):
    w = W["fp8_resident"]
    log("generating the fp8_resident bank (96 resident slots)")
    canon = _make_bank(w, 0)
    host = canon.to("cpu")
    dev = device_bank(canon)
    del canon
    torch.cuda.empty_cache()
    return host, dev


@pytest.mark.parametrize("T,n_sample", [(1, 1), (16, 16), (256, 256), (4096, 8), (16384, 8)])
def test_fp8_resident_full(ft, fp8_bank, T, n_sample):
    w = W["fp8_resident"]
    host, dev = fp8_bank
    li = _inputs(w, 0, T, bank=host)
    _check(ft, li, dev, n_sample=n_sample, label=f"fp8_resident T={T}", small_groups=4)
