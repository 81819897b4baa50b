"""ft_moe_layer_noalloc (the layer with the library's static device scratch instead of a workspace)
against ft_moe_layer (the same call with the caller's workspace) through the C ABI: two calls in a
row on one stream, the second with fewer tokens (or, once, more), on the one-kernel decode path and
on the four-call path.  Both calls run the same kernels on the same inputs, so every result matches
bit for bit; the outputs also meet the FFN tolerance against the oracle, and the status word is 0."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_ffn_close, device_bank, log

pytestmark = pytest.mark.gpu

CASES = {
    # one-kernel decode path: Q4_0 at the decode shape, MXFP4 with a shared expert and partial residency
    "q4_0_decode": (synth.WORKLOADS["decode_q4_0"].replace(layers=1, T=16), (16, 5)),
    "mxfp4_shared": (synth.Workload("noalloc_mx", 72, T=16, d=256, E=8, k=2, I=128, fmt=synth.FMT_MXFP4, shared=True),
                     (16, 3)),
    # four calls (T > 16): route, permute, grouped FFN on GEMV and GEMM kernels, combine
    "bf16_calls": (synth.WORKLOADS["prefill_bf16_zipf"].replace(T=40, d=512, I=256, E=16, k=4), (40, 17)),
    # more tokens after fewer: the second call's counters lie where the first left h rows
    "mxfp4_grow": (synth.Workload("noalloc_mx", 72, T=16, d=256, E=8, k=2, I=128, fmt=synth.FMT_MXFP4, shared=True),
                   (3, 16)),
    # rows of 4096 (8 waves per block, FP8 block scales staged per item)
    "fp8_long_rows": (synth.Workload("noalloc_long", 73, T=16, d=4096, E=8, k=8, I=2048, fmt=synth.FMT_FP8_B128),
                      (16, 9)),
}


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_expert_ffn_wave_amd as ft
    return ft


def _results(layer, T):
    n = T * layer.k
    return {"ids": layer.ids[:T].cpu().numpy(), "w": layer.w[:T].cpu().numpy().view(np.uint32),
            "counts": layer.counts.cpu().numpy(), "offsets": layer.offsets.cpu().numpy(),
            "gather": layer.gather[:n].cpu().numpy(), "inv": layer.inv[:n].cpu().numpy(),
            "mask": layer.mask[:T].cpu().numpy(), "out": layer.out[:T].float().cpu().numpy()}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_layer(ft, name):
    w, Ts = CASES[name]
    li = synth.layer_inputs(w, layer=1, T=max(Ts))
    bank = device_bank(li.bank)
    slot = li.slot_of_expert.clone()
    if name.startswith("mxfp4"):
        slot[[1, 6]] = -1  # two experts not resident: their pairs go to the mask
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    for T in Ts:  # two calls in a row
        log(f"noalloc {name}: T={T}")
        logits, x = li.logits[:T].cuda().contiguous(), li.x[:T].cuda().contiguous()
        ref_layer = ft.MoELayer(bank, slot.cuda(), w.k, T, shared_slot=w.shared_slot)
        ref_layer.forward(logits, x)
        torch.cuda.synchronize()
        assert ref_layer.status_word() == 0
        ref = _results(ref_layer, T)
        na = ft.MoELayer(bank, slot.cuda(), w.k, T, shared_slot=w.shared_slot)
        for buf in (na.out, na.y_sorted, na.gather, na.inv):
            buf.fill_(0)
        na.forward_noalloc(logits, x, status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "status word of the allocation-free call"
        got = _results(na, T)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), f"{name} T={T}: {key} differs from ft_moe_layer"
        ora = oracle.layer(li.logits[:T], li.x[:T], li.bank, slot, w.k, shared_slot=w.shared_slot)
        assert np.array_equal(got["ids"], ora["ids"]) and np.array_equal(got["gather"], ora["gather"])
        assert np.array_equal(got["mask"].astype(np.uint32), ora["mask"])
        assert_ffn_close(got["out"], ora["out"], f"noalloc {name} T={T}")
        status.fill_(-7)


def test_noalloc_refuses_oversize(ft):
    """A layer whose workspace exceeds the static scratch is refused and enqueues nothing."""
    w = synth.WORKLOADS["prefill_bf16_zipf"].replace(T=4096, d=512, I=512, E=16, k=4)
    li = synth.layer_inputs(w, layer=0, T=4096)
    bank = device_bank(li.bank)
    layer = ft.MoELayer(bank, li.slot_of_expert.cuda(), w.k, 4096)
    assert ft.lib.ft_moe_layer_workspace(bank.ref, 4096, w.E, w.k, -1, 0) > ft.FT_NOALLOC_SCRATCH_BYTES
    with pytest.raises(ft.FtError, match="static scratch"):
        layer.forward_noalloc(li.logits.cuda(), li.x.cuda())
