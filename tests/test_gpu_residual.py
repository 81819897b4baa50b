"""The cold-expert residual path against the oracle: the device layer on a bank that holds only some
experts leaves the other pairs to the residual mask; the host residual computes those pairs from
the bank of every expert in host memory (device layout, packed on the GPU), and its merge into the
device output must equal the oracle layer with every expert resident, within the FFN tolerance.
The residual alone must equal the difference of the oracle's full and partial layers."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import WORKERS, assert_ffn_close, device_bank, log, run_gpu_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_expert_ffn_wave_amd as ft
    return ft


FMTS = [synth.FMT_BF16, synth.FMT_Q4_0, synth.FMT_MXFP4, synth.FMT_FP8_B128, synth.FMT_NVFP4]


def _case(fmt, T, shared):
    return synth.Workload("residual", 90 + fmt, T=T, d=256, E=16, k=4, I=128, fmt=fmt, zipf=True, n_resident=6,
                          shared=shared)


@pytest.mark.parametrize("out_bf16", [False, True], ids=["f32_out", "bf16_out"])
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: synth.FMT_NAMES[f])
def test_residual_completes_the_layer(ft, fmt, out_bf16):
    T = 24
    w = _case(fmt, T, shared=False)
    log(f"residual {synth.FMT_NAMES[fmt]} T={T} out_bf16={out_bf16}")
    li = synth.layer_inputs(w, layer=0, T=T)
    flags = ft.FT_OUT_BF16 if out_bf16 else 0
    g = run_gpu_layer(li, device_bank(li.bank), flags=flags)
    assert g["mask"].any(), "the case should leave pairs to the residual path"
    # every routed expert, expert e in slot e, in host memory in the device layout
    w_all = w.replace(n_resident=None, shared=False)
    canon_all = synth.make_bank(w_all, 0)
    host = device_bank(canon_all).to_pinned_host()
    ids = torch.from_numpy(g["ids"])
    wts = torch.from_numpy(g["w"])
    mask = torch.from_numpy(g["mask"].view(np.int32))
    res = ft.ft_moe_residual_host(host, li.x, ids, wts, mask, n_threads=8)
    out = torch.from_numpy(g["out"]).cuda()
    out = out.to(torch.bfloat16) if out_bf16 else out
    ft.ft_moe_residual_add(out, res.cuda(), flags=flags)
    torch.cuda.synchronize()
    merged = out.float().cpu().numpy()
    full_slots = torch.arange(w.E, dtype=torch.int32)
    ora_full = oracle.layer(li.logits, li.x, canon_all, full_slots, w.k, workers=WORKERS)
    ora_part = oracle.layer(li.logits, li.x, li.bank, li.slot_of_expert, w.k, shared_slot=w.shared_slot,
                            workers=WORKERS)
    assert np.array_equal(g["mask"], ora_part["mask"])
    assert_ffn_close(merged, ora_full["out"], f"{synth.FMT_NAMES[fmt]}: device layer + host residual")
    assert_ffn_close(res.numpy(), ora_full["out"] - ora_part["out"], f"{synth.FMT_NAMES[fmt]}: host residual")
    untouched = g["mask"] == 0
    assert np.array_equal(res.numpy()[untouched], np.zeros((int(untouched.sum()), w.d), np.float32))


def test_residual_nothing_masked_and_everything_masked(ft):
    """No masked pair: the residual is zero.  Nothing resident: the residual alone is the layer."""
    w = _case(synth.FMT_Q4_0, 8, shared=False)
    li = synth.layer_inputs(w, layer=1, T=8)
    canon_all = synth.make_bank(w.replace(n_resident=None), 1)
    host = device_bank(canon_all).to_pinned_host()
    ids, wts = oracle.route(li.logits, w.k)
    ids_t, w_t = torch.from_numpy(ids), torch.from_numpy(wts)
    zero = torch.zeros(8, dtype=torch.int32)
    assert torch.count_nonzero(ft.ft_moe_residual_host(host, li.x, ids_t, w_t, zero)) == 0
    allm = torch.full((8,), (1 << w.k) - 1, dtype=torch.int32)
    res = ft.ft_moe_residual_host(host, li.x, ids_t, w_t, allm).numpy()
    ora = oracle.layer(li.logits, li.x, canon_all, torch.arange(w.E, dtype=torch.int32), w.k, workers=WORKERS)
    assert_ffn_close(res, ora["out"], "everything masked")
