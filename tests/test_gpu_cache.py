"""GPU parity of the global LRU expert cache, called through the C ABI: the update step against the
oracle bit for bit over sequences of steps, the fill byte for byte against the source bank, and
layer steps that copy experts in on a second stream while the grouped FFN runs, against the oracle
layer on the same inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_ffn_close, compare_layer, device_bank, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_expert_ffn_wave_amd as ft
    return ft


def _u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def _check_state(cache, st, label):
    assert np.array_equal(cache.slot_of_expert.cpu().numpy(), st.slot_of_expert), f"{label}: slot_of_expert"
    assert np.array_equal(cache.expert_of_slot.cpu().numpy(), st.expert_of_slot), f"{label}: expert_of_slot"
    assert np.array_equal(_u32(cache.last_use), st.last_use), f"{label}: last_use"
    assert np.array_equal(_u32(cache.tick), st.tick), f"{label}: tick"


# (E, n_slots, T, k, max_loads, steps, preload)
UPDATE_CASES = [
    (8, 1, 2, 2, 1, 40, False),
    (64, 16, 4, 4, 3, 60, False),
    (128, 32, 8, 8, 8, 60, False),
    (256, 96, 16, 8, 8, 40, True),
    (256, 96, 1, 8, 96, 30, False),
    (1024, 1000, 64, 8, 64, 12, False),
    (1024, 16, 64, 8, 16, 12, True),
    (32, 32, 8, 2, 32, 30, False),
    (16, 8, 4, 2, 0, 10, True),
    (1, 1, 4, 1, 1, 6, False),            # one expert, one slot
    (1024, 1024, 128, 8, 1024, 4, False),  # the largest tables, every slot loadable in one step
]
# (E, n_slots, T, k, max_loads, steps, load fraction)
FRACTION_CASES = [(64, 16, 4, 4, 16, 40, 0.5), (256, 96, 16, 8, 32, 30, 0.37), (128, 32, 8, 8, 8, 30, 1.0),
                  (32, 8, 8, 2, 8, 30, 0.1)]


@pytest.mark.parametrize("case", UPDATE_CASES, ids=lambda c: "E{}_S{}_T{}_k{}_ml{}_n{}_{}".format(*c))
def test_cache_update_matches_oracle(ft, case):
    E, S, T, k, ml, steps, preload = case
    log(f"cache update E={E} S={S} T={T} k={k} max_loads={ml} steps={steps} preload={preload}")
    seed = 7000 + E + 3 * S + ml
    st = oracle.CacheState(E, S)
    cache = ft.ExpertCache(E, S, ml)
    if preload:  # a consistent non-empty start: S random experts with random last uses
        rng = np.random.default_rng(seed)
        held = rng.permutation(E)[: min(S, E)]
        st.expert_of_slot[: len(held)] = held
        st.slot_of_expert[held] = np.arange(len(held), dtype=np.int32)
        st.last_use[:] = rng.integers(0, 5, size=S).astype(np.uint32)
        st.tick[0] = 5
        cache.slot_of_expert.copy_(torch.from_numpy(st.slot_of_expert))
        cache.expert_of_slot.copy_(torch.from_numpy(st.expert_of_slot))
        cache.last_use.copy_(torch.from_numpy(st.last_use.view(np.int32)))
        cache.tick.copy_(torch.from_numpy(st.tick.view(np.int32)))
    total_loads = 0
    for step in range(steps):
        counts = synth.zipf_counts(E, T, k, seed, step)
        if step % 7 == 3:
            counts[:] = 0   # a step without tokens
        cs_ref, loads_ref = oracle.cache_update(counts, st, ml)
        cs, loads, nl = cache.update(torch.from_numpy(counts).cuda())
        torch.cuda.synchronize()
        n = int(nl.item())
        label = f"step {step}"
        assert n == len(loads_ref), f"{label}: {n} loads, oracle {len(loads_ref)}"
        assert np.array_equal(loads[:n].cpu().numpy(), loads_ref), f"{label}: loads"
        assert np.array_equal(cs.cpu().numpy(), cs_ref), f"{label}: compute_slot"
        _check_state(cache, st, label)
        total_loads += n
    log(f"  ok: {total_loads} loads over {steps} steps")


@pytest.mark.parametrize("case", FRACTION_CASES, ids=lambda c: "E{}_S{}_T{}_k{}_ml{}_n{}_q{}".format(*c))
def test_cache_update_load_fraction(ft, case):
    """The load fraction and the table of this step's loads, bit for bit against the oracle."""
    E, S, T, k, ml, steps, q = case
    log(f"cache update with load fraction {q}: E={E} S={S}")
    st = oracle.CacheState(E, S)
    cache = ft.ExpertCache(E, S, ml, load_fraction=q)
    for step in range(steps):
        counts = synth.zipf_counts(E, T, k, 9000 + E + S, step)
        cs_ref, loads_ref, ls_ref = oracle.cache_update(counts, st, ml, q, with_load_slot=True)
        cs, loads, nl = cache.update(torch.from_numpy(counts).cuda())
        torch.cuda.synchronize()
        n = int(nl.item())
        assert n == len(loads_ref) and np.array_equal(loads[:n].cpu().numpy(), loads_ref), f"step {step}: loads"
        assert np.array_equal(cs.cpu().numpy(), cs_ref), f"step {step}: compute_slot"
        assert np.array_equal(cache.load_slot.cpu().numpy(), ls_ref), f"step {step}: load_slot"
        _check_state(cache, st, f"step {step}")


def _slot_arrays(bank, s: int):
    """Byte views of every array of slot s of a bank (public device layout)."""
    import routed_expert_ffn_wave_amd as ft
    out = []
    for which, arr in enumerate((bank.w13, bank.w2, bank.s13, bank.s2)):
        if arr is None:
            continue
        a = arr.view(torch.uint8).reshape(-1)
        if bank.fmt == ft.FT_W_NVFP4 and which >= 2:   # block scales per slot, then one fp32 per slot
            rows, K = (2 * bank.I, bank.d) if which == 2 else (bank.d, bank.I)
            blk = rows * (K // 32) * 2
            out.append(a[blk * s: blk * (s + 1)])
            out.append(a[blk * bank.n_slots + 4 * s: blk * bank.n_slots + 4 * s + 4])
        else:
            per = ft.ft_moe_bank_bytes(bank.fmt, 1, bank.d, bank.I, which)
            out.append(a[per * s: per * (s + 1)])
    return out


def _check_resident_bytes(cache, full, dst, label):
    eos = cache.expert_of_slot.cpu().tolist()
    for s, e in enumerate(eos):
        if e < 0:
            continue
        for i, (a, b) in enumerate(zip(_slot_arrays(dst, s), _slot_arrays(full, e))):
            assert torch.equal(a, b), f"{label}: slot {s} (expert {e}) array part {i} differs"
    return sum(e >= 0 for e in eos)


FILL_FMTS = [synth.FMT_BF16, synth.FMT_Q4_0, synth.FMT_MXFP4, synth.FMT_FP8_B128, synth.FMT_NVFP4]


@pytest.mark.parametrize("source", ["pinned", "device"])
@pytest.mark.parametrize("fmt", FILL_FMTS, ids=lambda f: synth.FMT_NAMES[f])
def test_cache_fill_bytes(ft, fmt, source):
    """After each step's update and fill, every occupied slot holds its expert's bytes exactly."""
    E, S, d, I, ml = 12, 5, 256, 128, 3
    log(f"cache fill {synth.FMT_NAMES[fmt]} from {source} memory")
    w = synth.Workload("cache_fill", 80, T=8, d=d, E=E, k=2, I=I, fmt=fmt)
    full = device_bank(synth.make_bank(w, 0))    # expert e in slot e
    src = full.to_pinned_host() if source == "pinned" else full
    dst = ft.DeviceBank.empty(fmt, S, d, I)
    for t in (dst.w13, dst.w2, dst.s13, dst.s2):
        if t is not None:
            t.fill_(0xA5)
    cache = ft.ExpertCache(E, S, ml)
    side = torch.cuda.Stream()
    loads = 0
    for step in range(10):
        counts = torch.from_numpy(synth.zipf_counts(E, 3, 2, 81, step)).cuda()
        _, _, nl = cache.update(counts)
        side.wait_stream(torch.cuda.current_stream())
        cache.fill(src, dst, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        loads += int(nl.item())
        _check_resident_bytes(cache, full, dst, f"step {step}")
    assert loads > S, "the sequence should evict"
    log(f"  ok: {loads} loads")


def test_cache_fill_full_shape(ft):
    """The 284B-class expert shape (d=7168, I=2048, FP8-B128, 44 MB per expert) from pinned host
    memory: 16 experts on the host, 6 slots, 4 loads per step."""
    E, S, d, I, ml = 16, 6, 7168, 2048, 4
    log("cache fill FP8-B128 d=7168 I=2048 from pinned memory")
    w = synth.Workload("cache_fill_full", 82, T=8, d=d, E=E, k=2, I=I, fmt=synth.FMT_FP8_B128)
    full = device_bank(synth.make_bank(w, 0, device="cuda"))
    src = full.to_pinned_host()
    dst = ft.DeviceBank.empty(w.fmt, S, d, I)
    cache = ft.ExpertCache(E, S, ml)
    side = torch.cuda.Stream()
    for step in range(5):
        counts = torch.from_numpy(synth.zipf_counts(E, 4, 2, 83, step)).cuda()
        cache.update(counts)
        side.wait_stream(torch.cuda.current_stream())
        cache.fill(src, dst, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        _check_resident_bytes(cache, full, dst, f"step {step}")
    log("  ok")


# (T, d, I, steps): few tokens run the GEMV kernels beside the fill; from 256 tokens every group
# runs on the GEMM kernels (the scaled-MFMA ones for MXFP4 and FP8-B128)
STREAM_SHAPES = {"gemv_T16": (16, 256, 128, 8), "gemm_T300": (300, 512, 256, 4)}


@pytest.mark.parametrize("shape", list(STREAM_SHAPES))
@pytest.mark.parametrize("fmt", [synth.FMT_Q4_0, synth.FMT_MXFP4, synth.FMT_FP8_B128],
                         ids=lambda f: synth.FMT_NAMES[f])
def test_cache_streamed_layer_steps(ft, fmt, shape):
    """Layer steps with the cache: route, permute, cache update; the fill on a second stream beside
    the grouped FFN and combine, which use this step's compute_slot.  Each step's ids, permutation,
    mask and outputs equal the oracle layer's on the full bank with the oracle cache's compute_slot."""
    T, d, I, steps = STREAM_SHAPES[shape]
    E, S, k, ml = 16, 6, 4, 3
    w = synth.Workload("cache_layer", 84, T=T, d=d, E=E, k=k, I=I, fmt=fmt, zipf=True)
    log(f"streamed layer steps {synth.FMT_NAMES[fmt]} T={T} d={d} I={I}")
    canon_full = synth.make_bank(w, 0)
    full = device_bank(canon_full)
    src = full.to_pinned_host()
    dst = ft.DeviceBank.empty(fmt, S, w.d, w.I)
    cache = ft.ExpertCache(E, S, ml)
    st = oracle.CacheState(E, S)
    side = torch.cuda.Stream()
    x_host = synth.activations(w, 0, T)
    x = x_host.cuda()
    for step in range(steps):
        logits_host = synth.step_logits(w, step, T)
        ids, wts = ft.ft_moe_route(logits_host.cuda(), k)
        counts, offsets, gather, inv = ft.ft_moe_permute(ids, E)
        cs, loads, nl = cache.update(counts)
        side.wait_stream(torch.cuda.current_stream())
        cache.fill(src, dst, stream=side)
        y, _ = ft.ft_moe_grouped_ffn(dst, cs, x, k, offsets, gather)
        out, mask = ft.ft_moe_combine(y, None, ids, wts, inv, cs, w.d)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        cs_ref, loads_ref = oracle.cache_update(counts.cpu().numpy(), st, ml)
        assert np.array_equal(cs.cpu().numpy(), cs_ref), f"step {step}: compute_slot"
        assert np.array_equal(loads[: int(nl.item())].cpu().numpy(), loads_ref), f"step {step}: loads"
        slot_ref = torch.from_numpy(np.where(cs_ref >= 0, np.arange(E), -1).astype(np.int32))
        li = synth.LayerInputs(w, 0, T, logits_host, x_host, slot_ref, canon_full)
        n = T * k
        g = dict(ids=ids.cpu().numpy(), w=wts.cpu().numpy(), counts=counts.cpu().numpy(),
                 offsets=offsets.cpu().numpy(), gather=gather[:n].cpu().numpy(), inv=inv[:n].cpu().numpy(),
                 y_sorted=y[:n], y_shared=None, out=out.float().cpu().numpy(),
                 mask=mask.cpu().numpy().astype(np.uint32))
        compare_layer(li, g, label=f"streamed step {step} ({int(nl.item())} loads, "
                                   f"{int((cs_ref >= 0).sum())} resident for compute)")
    _check_state(cache, st, "final")


def test_cache_step_graph_replay(ft):
    """A whole cache step (route, permute, cache update; the fill on a second stream beside the
    grouped FFN and combine) captured once into a HIP graph and replayed step after step with new
    logits copied in between: after every replay the outputs and the cache state equal those of the
    same steps run eagerly on a second cache from the same start, bit for bit."""
    E, S, T, k, ml, steps = 16, 6, 16, 4, 3, 6
    w = synth.Workload("cache_graph", 85, T=T, d=256, E=E, k=k, I=128, fmt=synth.FMT_Q4_0, zipf=True)
    log("cache step graph replay")
    full = device_bank(synth.make_bank(w, 0))
    src = full.to_pinned_host()
    x = synth.activations(w, 0, T).cuda()
    seq = [synth.step_logits(w, i, T).cuda() for i in range(steps)]
    dev = "cuda"

    def make():
        dst = ft.DeviceBank.empty(w.fmt, S, w.d, w.I)
        cache = ft.ExpertCache(E, S, ml)
        b = dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev),
                 ids=torch.empty(T, k, dtype=torch.int32, device=dev),
                 w=torch.empty(T, k, dtype=torch.float32, device=dev),
                 counts=torch.empty(E, dtype=torch.int32, device=dev),
                 offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                 gather=torch.empty(T * k, dtype=torch.int32, device=dev),
                 inv=torch.empty(T * k, dtype=torch.int32, device=dev),
                 pws=torch.empty(max(ft.ft_moe_permute_workspace(T, E, k), 16), dtype=torch.uint8, device=dev),
                 y=torch.empty(T * k, w.d, dtype=torch.bfloat16, device=dev),
                 fws=torch.empty(max(ft.ft_moe_grouped_ffn_workspace(dst, T, E, k), 256), dtype=torch.uint8,
                                 device=dev),
                 out=torch.empty(T, w.d, dtype=torch.float32, device=dev),
                 mask=torch.empty(T, dtype=torch.int32, device=dev))
        return dst, cache, b, torch.cuda.Stream()

    def step(dst, cache, b, side):
        main = torch.cuda.current_stream()
        ft.ft_moe_route(b["logits"], k, ids=b["ids"], w=b["w"])
        ft.ft_moe_permute(b["ids"], E, counts=b["counts"], offsets=b["offsets"], gather=b["gather"], inv=b["inv"],
                          ws=b["pws"])
        cs, _, _ = cache.update(b["counts"])
        side.wait_stream(main)
        cache.fill(src, dst, stream=side)
        ft.ft_moe_grouped_ffn(dst, cs, x, k, b["offsets"], b["gather"], y_sorted=b["y"], ws=b["fws"])
        ft.ft_moe_combine(b["y"], None, b["ids"], b["w"], b["inv"], cs, w.d, out=b["out"], residual_mask=b["mask"])
        main.wait_stream(side)

    def snapshot(cache, b):
        return [t.clone() for t in (b["out"], b["mask"], cache.compute_slot, cache.slot_of_expert,
                                    cache.expert_of_slot, cache.last_use, cache.tick, cache.n_loads)]

    A = make()
    eager = []
    for i in range(steps):
        A[2]["logits"].copy_(seq[i])
        step(*A)
        torch.cuda.synchronize()
        eager.append(snapshot(A[1], A[2]))

    B = make()
    dst, cache, b, side = B
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up outside the capture, then back to the empty start
        b["logits"].copy_(seq[0])
        step(*B)
        torch.cuda.synchronize()
        cache.slot_of_expert.fill_(-1)
        cache.expert_of_slot.fill_(-1)
        cache.last_use.zero_()
        cache.tick.zero_()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step(*B)
    torch.cuda.synchronize()
    for i in range(steps):
        b["logits"].copy_(seq[i])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(cache, b)
        names = ("out", "mask", "compute_slot", "slot_of_expert", "expert_of_slot", "last_use", "tick", "n_loads")
        for n, g_, e_ in zip(names, got, eager[i]):
            assert torch.equal(g_, e_), f"replay {i}: {n} differs from the eager step"
    assert int(cache.tick.item()) == steps
    log(f"  ok: {steps} replays")


@pytest.mark.parametrize("fmt", [synth.FMT_Q4_0, synth.FMT_FP8_B128], ids=lambda f: synth.FMT_NAMES[f])
def test_coexecuted_steps(ft, fmt):
    """The bandwidth-adaptive split in one step: a fraction of the cold experts is copied to the GPU
    and computed there after the copy, the rest on the host at the same time.  Per step: route,
    permute, cache update (load fraction 0.5); the host reads ids, w and the updated slot table and
    computes the pairs whose expert has no slot, while the device runs the fill (second stream), the
    FFN of the experts resident before the step, then, after the fill, the FFN of the experts just
    loaded, and the combine over the updated table.  The merged output equals the oracle layer with
    every expert resident; the mask marks exactly the pairs the host computed."""
    import threading
    E, S, T, k, ml, steps, q = 16, 6, 16, 4, 4, 6, 0.5
    w = synth.Workload("coexec", 86 + fmt, T=T, d=256, E=E, k=k, I=128, fmt=fmt, zipf=True)
    log(f"co-executed steps {synth.FMT_NAMES[fmt]}")
    canon_full = synth.make_bank(w, 0)
    host = device_bank(canon_full).to_pinned_host()
    dst = ft.DeviceBank.empty(fmt, S, w.d, w.I)
    cache = ft.ExpertCache(E, S, ml, load_fraction=q)
    st = oracle.CacheState(E, S)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    x_host = synth.activations(w, 0, T)
    x = x_host.cuda()
    for step in range(steps):
        logits_host = synth.step_logits(w, step, T)
        ids, wts = ft.ft_moe_route(logits_host.cuda(), k)
        counts, offsets, gather, inv = ft.ft_moe_permute(ids, E)
        cs, loads, nl = cache.update(counts)
        ids_h, w_h, slots_h = ids.cpu(), wts.cpu(), cache.slot_of_expert.cpu()   # waits for the update
        res = {}
        th = threading.Thread(target=lambda: res.update(
            r=ft.ft_moe_residual_host(host, x_host, ids_h, w_h, None, n_threads=4, slot_of_expert=slots_h)))
        th.start()
        side.wait_stream(main)
        cache.fill(host, dst, stream=side)
        y, _ = ft.ft_moe_grouped_ffn(dst, cs, x, k, offsets, gather)
        main.wait_stream(side)
        ft.ft_moe_grouped_ffn(dst, cache.load_slot, x, k, offsets, gather, y_sorted=y)
        out, mask = ft.ft_moe_combine(y, None, ids, wts, inv, cache.slot_of_expert, w.d)
        th.join()
        ft.ft_moe_residual_add(out, res["r"].cuda())
        torch.cuda.synchronize()
        cs_ref, loads_ref, ls_ref = oracle.cache_update(counts.cpu().numpy(), st, ml, q, with_load_slot=True)
        assert np.array_equal(cs.cpu().numpy(), cs_ref) and np.array_equal(cache.load_slot.cpu().numpy(), ls_ref)
        m = mask.cpu().numpy().view(np.uint32)
        want = ((slots_h.numpy()[ids_h.numpy()] < 0).astype(np.uint32) << np.arange(k, dtype=np.uint32)).sum(axis=1)
        assert np.array_equal(m, want.astype(np.uint32)), f"step {step}: mask"
        ora = oracle.layer(logits_host, x_host, canon_full, torch.arange(E, dtype=torch.int32), k)
        assert np.array_equal(ids_h.numpy(), ora["ids"])
        assert_ffn_close(out.cpu().numpy(), ora["out"], f"step {step}: co-executed layer")
        log(f"  step {step}: {int(nl.item())} loads computed on the GPU this step, "
            f"{int(sum(bin(int(v)).count('1') for v in m))} pairs on the host")


def test_cache_fill_refuses_pageable_source(ft):
    """A source bank in ordinary (pageable) host memory is refused before any launch."""
    E, S, d, I = 4, 2, 256, 128
    fmt = synth.FMT_Q4_0
    arrs = [torch.zeros(ft.ft_moe_bank_bytes(fmt, E, d, I, which), dtype=torch.uint8) for which in range(4)]
    src = ft.DeviceBank(fmt, E, d, I, *arrs)
    dst = ft.DeviceBank.empty(fmt, S, d, I)
    cache = ft.ExpertCache(E, S, 1)
    with pytest.raises(ft.FtError, match="neither pinned host memory nor device memory"):
        cache.fill(src, dst)
