"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle on the same seeded
inputs.  Routing ids, counts, offsets, permutation, residual mask and dequantised weights must match
bit for bit; routing weights within 1e-6; FFN rows and layer outputs within rel-L2 5e-3 and
max-abs 3e-2 * max|ref|."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import compare_layer, device_bank, log, run_gpu_layer, WTOL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ft():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import routed_expert_ffn_wave_amd as ft
    return ft


def _logits(kind, T, E, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "ties":
        L = torch.randint(-3, 4, (T, E), generator=g).float() * 0.5
        L[torch.rand(T, E, generator=g) < 0.05] = float("-inf")
        L[:, 0] = torch.where(torch.rand(T, generator=g) < 0.3, torch.tensor(-0.0), L[:, 0])
        # keep at least k finite per row: the first column is finite
        return L
    L = torch.randn(T, E, generator=g)
    if kind == "zipf":
        L += -1.1 * torch.log(torch.randperm(E, generator=g).double() + 1).float()
    if kind == "wide":
        L *= 30.0
    return L


# (T, d, E, k): one token tile to many, E below, at and past the 64-expert tiles, K tails of 32
ROUTE_PROJ_CASES = [(16, 256, 8, 2), (8, 2048, 128, 8), (37, 512, 40, 6), (300, 7168, 256, 8), (5, 96, 512, 32),
                    (1, 2048, 128, 8), (4096, 2048, 128, 8)]


@pytest.mark.parametrize("T,d,E,k", ROUTE_PROJ_CASES)
def test_route_proj(ft, T, d, E, k):
    """Router projection + route in one launch.  Logits within the rounding bound of an fp32 sum
    of d products against the oracle's fp64 dot products; ids bit for bit (weights within WTOL,
    as for ft_moe_route) what the oracle's route gives for the GPU's own fp32 logits; the chosen
    experts a top-k of the fp64 logits within that bound.  A second call with a smaller T reuses the workspace."""
    w = synth.Workload("route_proj", 90, T=T, d=d, E=E, k=k, I=64, fmt=synth.FMT_BF16)
    x = synth.activations(w, 0, T, device="cuda")
    wr = synth.router_rows(w, 0, device="cuda")
    log(f"route_proj T={T} d={d} E={E} k={k}")
    ws = torch.zeros(max(ft.ft_moe_route_proj_workspace(T), 16), dtype=torch.uint8, device="cuda")
    for TT in (T, max(1, T // 3)):
        lg, ids, wt = ft.ft_moe_route_proj(x[:TT].contiguous(), wr, k, ws=ws)
        torch.cuda.synchronize()
        g = lg.cpu().numpy().astype(np.float64)
        ref = oracle.router_logits(x[:TT].cpu(), wr.cpu())
        xa = np.abs(oracle.bf16_to_f32(x[:TT].cpu())).astype(np.float64)
        wa = np.abs(oracle.bf16_to_f32(wr.cpu())).astype(np.float64)
        bound = d * 2.0 ** -24 * (xa @ wa.T) + 1e-30
        err = np.abs(g - ref)
        assert np.all(err <= bound), f"logit error {err.max()} over bound at {np.unravel_index(np.argmax(err - bound), err.shape)}"
        oids, ow = oracle.route(lg.cpu(), k)
        assert np.array_equal(ids.cpu().numpy(), oids)
        assert np.abs(wt.cpu().numpy() - ow).max() <= WTOL
        ids_np = ids.cpu().numpy()
        for t in range(TT):
            chosen = np.zeros(E, bool)
            chosen[ids_np[t]] = True
            if chosen.all():
                continue
            assert ref[t][chosen].min() >= ref[t][~chosen].max() - 2 * bound[t].max()
        assert not ws.any(), "the workspace must be left zero"


# (workload, T, flags): the one-launch path with the projection inside (decode shapes, a shared expert,
# partial residency, rows of 4096), and the two-launch path (T > 16, or the layer forced unfused)
LAYER_PROJ_CASES = {
    "q4_0_decode_T1": (synth.WORKLOADS["decode_q4_0"].replace(layers=1), 1, 0),
    "q4_0_decode_T8": (synth.WORKLOADS["decode_q4_0"].replace(layers=1), 8, 0),
    "tiny_bf16_T16": (synth.WORKLOADS["tiny_bf16"], 16, 0),
    "mxfp4_shared_T5": (synth.WORKLOADS["mxfp4_shared"].replace(d=512, I=256, E=32, k=4), 5, 0),
    "fp8_resident_T16": (synth.WORKLOADS["fp8_resident"].replace(d=512, I=256, E=32, k=4, n_resident=12), 16, 0),
    "fp8_long_rows_T16": (synth.Workload("long_rows", 72, T=16, d=4096, E=16, k=4, I=256, fmt=synth.FMT_FP8_B128,
                                         zipf=True), 16, 0),
    "q4_0_T40_two_launches": (synth.WORKLOADS["decode_q4_0"].replace(layers=1, T=40, d=512, I=256, E=16, k=4), 40, 0),
    "q4_0_T8_unfused": (synth.WORKLOADS["decode_q4_0"].replace(layers=1), 8, 8),
}


@pytest.mark.parametrize("name", list(LAYER_PROJ_CASES))
def test_layer_proj(ft, name):
    """ft_moe_layer_proj: the logits within the rounding bound of an fp32 sum of d products against
    the oracle's fp64 router projection; routing, permutation and mask bit for bit and FFN rows and
    outputs within the FFN tolerance against the oracle layer on the GPU's own logits; status word 0;
    a second call (the same workspace) repeats every bit."""
    w, T, flags = LAYER_PROJ_CASES[name]
    li = synth.layer_inputs(w, layer=2, T=T)
    wr = synth.router_rows(w, 2)
    bank = device_bank(li.bank)
    log(f"layer_proj {name}: T={T} d={w.d} E={w.E} k={w.k} flags={flags}")
    layer = ft.MoELayer(bank, li.slot_of_expert.cuda(), w.k, T, shared_slot=w.shared_slot, flags=flags)
    x, wr_d = li.x.cuda(), wr.cuda()
    out, mask = layer.forward_proj(x, wr_d)
    torch.cuda.synchronize()
    assert layer.status_word() == 0, "a wait of the fused kernel gave up"
    lg = layer.logits[:T].cpu()
    ref = oracle.router_logits(li.x, wr)
    xa = np.abs(oracle.bf16_to_f32(li.x)).astype(np.float64)
    wa = np.abs(oracle.bf16_to_f32(wr)).astype(np.float64)
    bound = w.d * 2.0 ** -24 * (xa @ wa.T) + 1e-30
    err = np.abs(lg.numpy().astype(np.float64) - ref)
    assert np.all(err <= bound), f"{name}: logit error {err.max()} over the bound"
    n = T * w.k
    g = dict(ids=layer.ids[:T].cpu().numpy(), w=layer.w[:T].cpu().numpy(), counts=layer.counts.cpu().numpy(),
             offsets=layer.offsets.cpu().numpy(), gather=layer.gather[:n].cpu().numpy(),
             inv=layer.inv[:n].cpu().numpy(), y_sorted=layer.y_sorted[:n],
             y_shared=None if layer.y_shared is None else layer.y_shared[:T],
             out=out.float().cpu().numpy(), mask=mask.cpu().numpy().astype(np.uint32))
    li_gpu = synth.LayerInputs(w, 2, T, lg, li.x, li.slot_of_expert, li.bank)
    compare_layer(li_gpu, g, label=f"layer_proj {name}")
    first_out, first_lg = g["out"].copy(), lg.clone()
    out2, _ = layer.forward_proj(x, wr_d)
    torch.cuda.synchronize()
    assert layer.status_word() == 0
    assert torch.equal(layer.logits[:T].cpu(), first_lg), f"{name}: logits not repeatable"
    assert np.array_equal(out2.float().cpu().numpy().view(np.uint32), first_out.view(np.uint32)), \
        f"{name}: output not repeatable"


ROUTE_CASES = [(1, 8, 2, "normal"), (37, 8, 2, "ties"), (64, 10, 4, "ties"), (300, 128, 8, "normal"),
               (513, 256, 8, "zipf"), (64, 1024, 32, "ties"), (5, 32, 32, "normal"), (33, 7, 1, "ties"),
               (20, 1, 1, "normal"), (100, 65, 8, "wide"), (16384, 256, 8, "zipf")]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route(ft, T, E, k, kind):
    L = _logits(kind, T, E, 1000 + T + E + k)
    ids, w = ft.ft_moe_route(L.cuda(), k)
    torch.cuda.synchronize()
    rid, rw = oracle.route(L, k)
    assert np.array_equal(ids.cpu().numpy(), rid)
    wg = w.cpu().numpy()
    finite = np.isfinite(rw)
    assert np.array_equal(np.isfinite(wg), finite)
    assert np.abs(wg[finite] - rw[finite]).max(initial=0) <= WTOL


PERMUTE_CASES = [(0, 8, 2, "rand"), (1, 8, 2, "rand"), (8, 128, 8, "rand"), (2048, 128, 8, "rand"),
                 (2049, 128, 8, "rand"), (4096, 128, 8, "skew"), (16384, 256, 8, "skew"), (600, 1024, 32, "rand"), (400, 1024, 32, "rand"),
                 (5000, 3, 3, "rand"), (3000, 1024, 1, "skew")]


@pytest.mark.parametrize("T,E,k,kind", PERMUTE_CASES)
def test_permute(ft, T, E, k, kind):
    g = torch.Generator().manual_seed(7 + T + E)
    if T == 0:
        ids = torch.zeros(0, k, dtype=torch.int32)
    else:
        ids = torch.argsort(torch.rand(T, E, generator=g), dim=1)[:, :k].to(torch.int32)
        if kind == "skew":
            hot = torch.arange(k, dtype=torch.int32)
            ids[: T * 3 // 4] = hot
    counts, offsets, gather, inv = ft.ft_moe_permute(ids.cuda(), E)
    torch.cuda.synchronize()
    rc, ro, rg, ri = oracle.permute(ids.numpy(), E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(gather.cpu().numpy(), rg)
    assert np.array_equal(inv.cpu().numpy(), ri)


def _bits_equal_nan_aware(a: np.ndarray, b: np.ndarray):
    na, nb = np.isnan(a), np.isnan(b)
    assert np.array_equal(na, nb), "NaN positions differ"
    assert np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("content", ["encoded", "random_bytes"])
def test_dequant_bit_exact(ft, fmt, content):
    d, I, n = 256, 384, 3
    if content == "encoded":
        w = synth.Workload("dq", 50, T=1, d=d, E=n, k=1, I=I, fmt=fmt)
        canon = synth.make_bank(w)
    else:  # every code and scale byte random: NaN/inf/subnormal scales, NaN codes, extreme exponents
        g = torch.Generator().manual_seed(60 + fmt)
        canon = synth.empty_bank(fmt, n, d, I)
        for t in (canon.w13, canon.w2):
            t.view(torch.uint8).copy_(torch.randint(0, 256, t.view(torch.uint8).shape, generator=g, dtype=torch.uint8))
        if fmt == 3:  # fp32 block scales: random finite positive normals of varied exponent
            for t in (canon.s13, canon.s2):
                t.copy_(torch.exp2(torch.randint(-40, 20, t.shape, generator=g).float()) *
                        (1 + torch.rand(t.shape, generator=g)))
        elif fmt in (2, 4):  # E8M0 bytes; NVFP4 e4m3 bytes and the fp32 matrix scale's bytes
            for t in (canon.s13, canon.s2):
                t.copy_(torch.randint(0, 256, t.shape, generator=g, dtype=torch.uint8))
    bank = device_bank(canon)
    for slot in range(n):
        for which, (rows, K) in enumerate(((2 * I, d), (d, I))):
            got = ft.ft_moe_dequant(bank, slot, which).cpu().numpy()
            codes = canon.w13[slot] if which == 0 else canon.w2[slot]
            sc = None if canon.s13 is None else (canon.s13[slot] if which == 0 else canon.s2[slot])
            ref = oracle.dequant(fmt, codes, sc, rows, K)
            _bits_equal_nan_aware(got, ref)


# ------------------------------------------------------------------------------------- whole layer, reduced sizes

def _small_workloads():
    W = synth.WORKLOADS
    return {
        "tiny_bf16": W["tiny_bf16"],
        "decode_q4_0": W["decode_q4_0"].replace(layers=1),
        "prefill_bf16_zipf": W["prefill_bf16_zipf"].replace(T=300, d=512, I=256, E=16, k=4),
        "mxfp4_shared": W["mxfp4_shared"].replace(T=200, d=512, I=256, E=32, k=4),
        "fp8_resident": W["fp8_resident"].replace(T=300, d=512, I=256, E=32, k=4, n_resident=12),
        "q4_0_prefill": W["decode_q4_0"].replace(T=150, d=512, I=256, E=16, k=4, layers=1),
        "nvfp4_decode": W["nvfp4_decode"].replace(layers=1),
        "nvfp4_prefill": W["nvfp4_decode"].replace(T=150, d=512, I=256, E=16, k=4, layers=1),
        # the shared expert's group on the bf16 and FP8 GEMM kernels (T >= 256: every group on them)
        "bf16_shared": W["mxfp4_shared"].replace(fmt=synth.FMT_BF16, T=300, d=512, I=256, E=32, k=4),
        "fp8_shared": W["mxfp4_shared"].replace(fmt=synth.FMT_FP8_B128, T=300, d=512, I=256, E=32, k=4),
    }


SMALL = _small_workloads()


@pytest.mark.parametrize("path", ["auto", "gemv", "gemm", "calls", "widen"])
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(ft, name, path):
    """ft_moe_layer with each FFN path (fused decode kernels where T <= 16), and the four calls;
    "widen": every group on the GEMM kernels with MXFP4 / FP8 weights widened to bf16 (the other
    formats run their usual GEMM kernels)."""
    w = SMALL[name]
    flags = {"auto": 0, "gemv": ft.FT_PATH_GEMV, "gemm": ft.FT_PATH_GEMM, "calls": 0,
             "widen": ft.FT_PATH_GEMM | ft.FT_GEMM_WIDEN}[path]
    T = w.T if name in ("tiny_bf16", "decode_q4_0") else min(w.T, 40 if path == "gemv" else w.T)
    log(f"layer {name} T={T} path={path}")
    li = synth.layer_inputs(w, layer=0, T=T)
    g = run_gpu_layer(li, device_bank(li.bank), flags=flags, mode="calls" if path == "calls" else "layer")
    compare_layer(li, g, label=f"{name}/{path}")


FUSED_T = [1, 3, 8, 13, 16]


@pytest.mark.parametrize("T", FUSED_T)
def test_fused_layer_matches_calls(ft, T):
    """The fused kernel routes with the router kernel's routine, so routing, permutation and mask
    match the four calls bit for bit; its FFN sums run in another grouping, so FFN rows and outputs
    match within the FFN tolerance (and the oracle's).  A second fused run repeats every bit."""
    from gpu_util import assert_ffn_close
    w = SMALL["decode_q4_0"].replace(T=16)
    li = synth.layer_inputs(w, layer=3, T=T)
    bank = device_bank(li.bank)
    a = run_gpu_layer(li, bank, flags=ft.FT_PATH_GEMV, mode="layer")
    b = run_gpu_layer(li, bank, flags=ft.FT_PATH_GEMV, mode="calls")
    for key in ("ids", "counts", "offsets", "gather", "inv", "mask"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["w"].view(np.uint32), b["w"].view(np.uint32))
    assert_ffn_close(a["out"], b["out"], f"fused vs calls T={T}: out")
    assert_ffn_close(a["y_sorted"].float().cpu().numpy(), b["y_sorted"].float().cpu().numpy(),
                     f"fused vs calls T={T}: y_sorted")
    again = run_gpu_layer(li, bank, flags=ft.FT_PATH_GEMV, mode="layer")
    assert np.array_equal(a["out"].view(np.uint32), again["out"].view(np.uint32))
    compare_layer(li, a, label=f"fused T={T}")


@pytest.mark.parametrize("T", [1, 16])
@pytest.mark.parametrize("case", ["mxfp4_shared", "partial_residency", "one_expert_takes_all", "k_equals_E",
                                  "bf16_out", "tokens_with_nothing_resident"])
def test_fused_layer_cases(ft, case, T):
    w = EDGE.replace(T=16)
    flags = 0
    if case == "k_equals_E":
        w = w.replace(k=8)
    if case == "tokens_with_nothing_resident":
        w = w.replace(shared=False)
    li = synth.layer_inputs(w, layer=2, T=T)
    if case == "tokens_with_nothing_resident":
        # only experts 6 and 7 stay: tokens routed elsewhere combine nothing and get zero rows
        li.slot_of_expert = li.slot_of_expert.clone()
        li.slot_of_expert[:6] = -1
    if case == "one_expert_takes_all":
        li.logits[:, 5] += 100.0
    if case == "partial_residency":
        # experts 1, 4 and 6 leave the bank: their pairs go to the mask, the rest still combine
        li.slot_of_expert = li.slot_of_expert.clone()
        li.slot_of_expert[[1, 4, 6]] = -1
    bank = device_bank(li.bank)
    if case == "bf16_out":
        # the same fp32 sums as the fp32 output, rounded to nearest even
        layer = ft.MoELayer(bank, li.slot_of_expert.cuda(), w.k, T, shared_slot=w.shared_slot, out_bf16=True)
        out, _ = layer.forward(li.logits.cuda(), li.x.cuda())
        torch.cuda.synchronize()
        assert layer.status_word() == 0
        ref = run_gpu_layer(li, bank, mode="layer")
        ref_bf16 = torch.from_numpy(ref["out"]).to(torch.bfloat16)
        assert torch.equal(out.cpu(), ref_bf16)
        return
    g = run_gpu_layer(li, bank, flags=flags)
    compare_layer(li, g, label=f"fused {case} T={T}")


@pytest.mark.parametrize("T", [1, 16])
@pytest.mark.parametrize("unfused", [False, True])
def test_layer_slots_beyond_bank(ft, T, unfused):
    """Slot-table entries at or past the bank's n_slots count as not resident on both paths of
    ft_moe_layer: the result equals the oracle's with those entries set to -1."""
    w = EDGE.replace(T=16, shared=False)
    li = synth.layer_inputs(w, layer=4, T=T)
    bank = device_bank(li.bank)
    n_slots = li.bank.n_slots
    ref_slots = li.slot_of_expert.clone()
    ref_slots[[2, 5]] = -1
    li.slot_of_expert = li.slot_of_expert.clone()
    li.slot_of_expert[2] = n_slots
    li.slot_of_expert[5] = n_slots + 7
    g = run_gpu_layer(li, bank, flags=ft.FT_LAYER_UNFUSED if unfused else 0)
    li.slot_of_expert = ref_slots
    compare_layer(li, g, label=f"slots beyond bank T={T} unfused={unfused}")


@pytest.mark.parametrize("T", [1, 5, 16, 37])
def test_layer_small_sweep_fp8(ft, T):
    w = SMALL["fp8_resident"]
    li = synth.layer_inputs(w, layer=1, T=T)
    g = run_gpu_layer(li, device_bank(li.bank))
    compare_layer(li, g, label=f"fp8 sweep T={T}")


# ------------------------------------------------------------------------------------- degenerate cases

# rows longer than 2048 on the fused path: 8 waves per block, FP8 block scales of two 128-row
# blocks per item, every format at a reduced shape (the full-size tests cover FP8 and MXFP4 only)
LONG = synth.Workload("long_rows", 72, T=16, d=4096, E=16, k=4, I=256, fmt=synth.FMT_FP8_B128, zipf=True)
LONG_FMTS = [synth.FMT_BF16, synth.FMT_Q4_0, synth.FMT_MXFP4, synth.FMT_FP8_B128, synth.FMT_NVFP4]


@pytest.mark.parametrize("case", ["plain", "shared", "one_expert_takes_all"])
@pytest.mark.parametrize("T", [1, 5, 16])
@pytest.mark.parametrize("fmt", LONG_FMTS, ids=lambda f: synth.FMT_NAMES[f])
def test_fused_long_rows(ft, fmt, T, case):
    """The fused layer at d = 4096: against the oracle on every token, against the four calls
    within the FFN tolerance, and bit for bit on a second run."""
    from gpu_util import assert_ffn_close
    w = LONG.replace(fmt=fmt, shared=case == "shared")
    li = synth.layer_inputs(w, layer=1, T=T)
    if case == "one_expert_takes_all":   # one group of all T tokens
        li.logits[:, 5] += 100.0
    bank = device_bank(li.bank)
    label = f"long rows {synth.FMT_NAMES[fmt]} {case} T={T}"
    a = run_gpu_layer(li, bank, mode="layer")
    compare_layer(li, a, label=label)
    b = run_gpu_layer(li, bank, mode="calls")
    for key in ("ids", "counts", "offsets", "gather", "inv", "mask"):
        assert np.array_equal(a[key], b[key]), f"{label}: {key}"
    assert_ffn_close(a["out"], b["out"], f"{label}: fused vs calls")
    again = run_gpu_layer(li, bank, mode="layer")
    assert np.array_equal(a["out"].view(np.uint32), again["out"].view(np.uint32)), f"{label}: not repeatable"


EDGE = synth.Workload("edge", 70, T=33, d=256, E=8, k=2, I=128, fmt=synth.FMT_MXFP4, shared=True)


@pytest.mark.parametrize("case", ["all_equal_logits", "k_equals_E", "k1", "T1", "one_expert_takes_all", "x_zero"])
def test_layer_degenerate(ft, case):
    w, T = EDGE, EDGE.T
    if case == "k_equals_E":
        w = EDGE.replace(k=8)
    elif case == "k1":
        w = EDGE.replace(k=1)
    elif case == "T1":
        T = 1
    li = synth.layer_inputs(w, layer=0, T=T)
    if case == "all_equal_logits":
        li.logits = torch.zeros(T, w.E)
    elif case == "one_expert_takes_all":
        li.logits[:, 3] += 100.0
    elif case == "x_zero":
        li.x = torch.zeros_like(li.x)
    bank = device_bank(li.bank)
    for flags in (0, ft.FT_PATH_GEMV, ft.FT_PATH_GEMM):
        g = run_gpu_layer(li, bank, flags=flags)
        if case == "x_zero":
            assert (g["out"] == 0).all()
        compare_layer(li, g, label=f"edge {case} flags={flags}")


def test_layer_nothing_resident(ft):
    """Every routed expert missing from the bank: only the shared expert contributes and every token
    carries all k mask bits."""
    li = synth.layer_inputs(EDGE, layer=0)
    li.bank = li.bank.slot(EDGE.E)                     # a one-slot bank holding the shared expert
    li.slot_of_expert = torch.full((EDGE.E,), -1, dtype=torch.int32)
    li.workload = EDGE.replace(E=EDGE.E)               # same shape; shared expert now in slot 0
    bank = device_bank(li.bank)
    layer = ft.MoELayer(bank, li.slot_of_expert.cuda(), EDGE.k, EDGE.T, shared_slot=0)
    out, mask = layer.forward(li.logits.cuda(), li.x.cuda())
    torch.cuda.synchronize()
    ora = oracle.layer(li.logits, li.x, li.bank, li.slot_of_expert, EDGE.k, shared_slot=0)
    assert (ora["mask"] == (1 << EDGE.k) - 1).all()
    assert np.array_equal(mask.cpu().numpy().astype(np.uint32), ora["mask"])
    from gpu_util import assert_ffn_close
    assert_ffn_close(out.cpu().numpy(), ora["out"], "nothing resident: out")


def test_t_zero_is_noop(ft):
    w = SMALL["tiny_bf16"]
    li = synth.layer_inputs(w, T=4)
    bank = device_bank(li.bank)
    layer = ft.MoELayer(bank, li.slot_of_expert.cuda(), w.k, 0)
    out, mask = layer.forward(li.logits[:0].cuda(), li.x[:0].cuda())
    torch.cuda.synchronize()
    assert out.shape == (0, w.d) and mask.shape == (0,)
    assert (layer.counts.cpu() == 0).all() and (layer.offsets.cpu() == 0).all()


def test_repeatable_bit_for_bit(ft):
    w = SMALL["prefill_bf16_zipf"]
    li = synth.layer_inputs(w, T=300)
    bank = device_bank(li.bank)
    a = run_gpu_layer(li, bank)
    b = run_gpu_layer(li, bank)
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32))
    assert torch.equal(a["y_sorted"], b["y_sorted"])


def test_graph_capture_replays(ft):
    """The four calls enqueue only, so a graph of one layer replays to the eager result."""
    w = SMALL["decode_q4_0"]
    li = synth.layer_inputs(w, T=8)
    bank = device_bank(li.bank)
    layer = ft.MoELayer(bank, li.slot_of_expert.cuda(), w.k, 8)
    logits, x = li.logits.cuda(), li.x.cuda()
    out, _ = layer.forward(logits, x)
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
    for _ in range(3):
        layer.out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, eager)


@pytest.mark.parametrize("unfused", [False, True])
def test_layer_nan_row_wide_router(ft, unfused):
    """A token whose logits are all NaN (unspecified input) with E = 512, where routing runs one
    token per wave and gives that token no valid expert: the layer still completes with status 0,
    the token carries every mask bit and a zero output row, and every other token matches the
    oracle (run with that row replaced by zeros; tokens are routed independently)."""
    from gpu_util import assert_ffn_close
    w = synth.Workload("nan_row", 71, T=6, d=256, E=512, k=8, I=128, fmt=synth.FMT_BF16)
    li = synth.layer_inputs(w, layer=0)
    bad = 2
    li.logits = li.logits.clone()
    li.logits[bad] = float("nan")
    bank = device_bank(li.bank)
    layer = ft.MoELayer(bank, li.slot_of_expert.cuda(), w.k, w.T,
                        flags=ft.FT_LAYER_UNFUSED if unfused else 0)
    out, mask = layer.forward(li.logits.cuda(), li.x.cuda())
    torch.cuda.synchronize()
    assert layer.status_word() == 0
    out, mask = out.cpu().numpy(), mask.cpu().numpy().astype(np.uint32)
    assert mask[bad] == (1 << w.k) - 1
    assert (out[bad] == 0).all()
    L0 = li.logits.clone()
    L0[bad] = 0.0
    ora = oracle.layer(L0, li.x, li.bank, li.slot_of_expert, w.k)
    keep = np.arange(w.T) != bad
    assert np.array_equal(layer.ids[:w.T].cpu().numpy()[keep], ora["ids"][keep])
    assert np.array_equal(mask[keep], ora["mask"][keep])
    assert_ffn_close(out[keep], ora["out"][keep], f"nan row unfused={unfused}: other tokens")


def test_two_host_threads(ft):
    """Launch code called from two host threads at once: layers of two shapes (different LDS sizes of
    the one-kernel decode path, and the GEMV and GEMM kernels of the four calls), repeated.  First
    both threads run the one-kernel path on one stream (the device runs them in turn; the host-side
    launch facts are shared between the threads); then on two streams, one thread the one-kernel path
    and the other the four calls.  Every result matches the oracle and every status word is 0."""
    import threading
    from gpu_util import assert_ffn_close
    shapes = {
        "q4_0_T8": SMALL["decode_q4_0"].replace(T=8),
        "mxfp4_T16": EDGE.replace(T=16),
        "bf16_T300": SMALL["prefill_bf16_zipf"],
    }
    inputs = {n: synth.layer_inputs(w, layer=5) for n, w in shapes.items()}
    banks = {n: device_bank(li.bank) for n, li in inputs.items()}
    refs = {n: oracle.layer(li.logits, li.x, li.bank, li.slot_of_expert, li.workload.k,
                            shared_slot=li.workload.shared_slot) for n, li in inputs.items()}

    def run(name, mode, stream, results, reps=4):
        try:
            li = inputs[name]
            w = li.workload
            layer = ft.MoELayer(banks[name], li.slot_of_expert.cuda(), w.k, li.T, shared_slot=w.shared_slot, mode=mode)
            logits, x = li.logits.cuda(), li.x.cuda()
            torch.cuda.synchronize()
            outs = []
            with torch.cuda.stream(stream):  # the copies of each result are ordered after its layer call
                for _ in range(reps):
                    out, mask = layer.forward(logits, x)
                    outs.append((out.clone(), mask.clone()))
            stream.synchronize()
            results[name] = (outs, layer.status_word())
        except Exception as e:  # reported by the main thread
            results[name] = e

    for plan in ((("q4_0_T8", "layer", 0), ("mxfp4_T16", "layer", 0)),
                 (("q4_0_T8", "layer", 0), ("bf16_T300", "calls", 1))):
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        results = {}
        threads = [threading.Thread(target=run, args=(n, m, streams[si], results)) for n, m, si in plan]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        for name, mode, _ in plan:
            r = results[name]
            assert not isinstance(r, Exception), f"{name}: {r!r}"
            outs, status = r
            assert status == 0, f"{name}: status word {status}"
            ref = refs[name]
            for out, mask in outs:
                assert np.array_equal(mask.cpu().numpy().astype(np.uint32), ref["mask"]), name
                assert_ffn_close(out.float().cpu().numpy(), ref["out"], f"two threads {name} ({mode})")
            log(f"two threads: {name} ({mode}) ok over {len(outs)} calls")
