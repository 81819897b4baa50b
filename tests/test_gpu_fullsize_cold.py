"""Full-size GPU parity of the cold-expert machinery at the fp8_resident shape (T=16, d=7168, E=256,
k=8, I=2048, FP8-B128, 96 device slots): the workload's 96 resident experts copied in by the fill,
then layer steps with the expert cache (update, fill of the chosen experts on a second stream
beside the grouped FFN and combine) and the host residual of the masked pairs merged into the
output.  Each step: compute_slot and loads bit for bit against the oracle's cache step, the residual
mask consistent with compute_slot, every occupied slot holding its expert's bytes, and the merged
output of sampled tokens against the oracle layer with every expert resident."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import WORKERS, assert_ffn_close, log, sample_tokens
from test_gpu_fullsize import _make_bank

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_expert_ffn_wave_amd as ft
    return ft


def test_fp8_resident_cold_experts_full(ft):
    w = synth.WORKLOADS["fp8_resident"]
    T, S, ml, steps = 16, w.n_resident, 2, 3
    E, k = w.E, w.k
    canon = _make_bank(w.replace(n_resident=None), 0)           # all 256 experts, expert e in slot e
    packed = ft.ft_moe_pack_bank(canon.fmt, E, w.d, w.I, canon.w13, canon.w2, canon.s13, canon.s2)
    host = packed.to_pinned_host()
    canon_host = canon.to("cpu")
    del canon, packed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("fp8_resident cold experts: host banks ready")

    # start: the workload's resident set (slot table of the recipe), copied in by the fill
    table = synth.slot_table(w, 0).numpy()
    st = oracle.CacheState(E, S)
    st.slot_of_expert[:] = table
    for e in np.flatnonzero(table >= 0):
        st.expert_of_slot[table[e]] = e
    dst = ft.DeviceBank.empty(w.fmt, S, w.d, w.I)
    pre = ft.ExpertCache(E, S, S)
    pairs = np.stack([st.expert_of_slot, np.arange(S)], axis=1).astype(np.int32)
    pre.loads.copy_(torch.from_numpy(pairs))
    pre.n_loads.fill_(S)
    pre.fill(host, dst)
    cache = ft.ExpertCache(E, S, ml)
    cache.slot_of_expert.copy_(torch.from_numpy(st.slot_of_expert))
    cache.expert_of_slot.copy_(torch.from_numpy(st.expert_of_slot))
    torch.cuda.synchronize()

    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    x = synth.activations(w, 0, T, device="cuda")
    x_host = x.cpu()
    for step in range(steps):
        logits = synth.step_logits(w, step, T, device="cuda")
        ids, wts = ft.ft_moe_route(logits, k)
        counts, offsets, gather, inv = ft.ft_moe_permute(ids, E)
        cs, loads, nl = cache.update(counts)
        side.wait_stream(main)
        cache.fill(host, dst, stream=side)
        y, _ = ft.ft_moe_grouped_ffn(dst, cs, x, k, offsets, gather)
        out, mask = ft.ft_moe_combine(y, None, ids, wts, inv, cs, w.d)
        main.wait_stream(side)
        torch.cuda.synchronize()
        cs_ref, loads_ref = oracle.cache_update(counts.cpu().numpy(), st, ml)
        assert np.array_equal(cs.cpu().numpy(), cs_ref), f"step {step}: compute_slot"
        assert np.array_equal(loads[: int(nl.item())].cpu().numpy(), loads_ref), f"step {step}: loads"
        ids_h, m_h, cs_h = ids.cpu().numpy(), mask.cpu().numpy().view(np.uint32), cs_ref
        want_mask = ((cs_h[ids_h] < 0).astype(np.uint32) << np.arange(k, dtype=np.uint32)).sum(axis=1)
        assert np.array_equal(m_h, want_mask.astype(np.uint32)), f"step {step}: residual mask"
        eos = cache.expert_of_slot.cpu().numpy()
        for s in list(loads_ref[:, 1]) + [0, S - 1]:
            e = int(eos[s])
            for a, b in ((dst.w13, host.w13), (dst.w2, host.w2), (dst.s13, host.s13), (dst.s2, host.s2)):
                per = a.numel() // S
                assert torch.equal(a[per * s: per * (s + 1)].cpu(), b[per * e: per * (e + 1)]), f"slot {s}"
        res = ft.ft_moe_residual_host(host, x_host, ids.cpu(), wts.cpu(), mask.cpu(), n_threads=16)
        ft.ft_moe_residual_add(out, res.cuda())
        torch.cuda.synchronize()
        tokens = sample_tokens(T, 4, seed=101 + step)
        ora = oracle.layer(logits.cpu(), x_host, canon_host, torch.arange(E, dtype=torch.int32), k, tokens=tokens,
                           workers=WORKERS)
        assert np.array_equal(ids_h, ora["ids"]), f"step {step}: ids"
        tok = ora["tokens"]
        assert_ffn_close(out.cpu().numpy()[tok], ora["out"][tok], f"step {step}: device layer + cache + residual")
        log(f"  step {step}: {int(nl.item())} loads, {int((m_h != 0).sum())} tokens with cold pairs, "
            f"{int(sum(bin(int(v)).count('1') for v in m_h))} cold pairs; ok")
