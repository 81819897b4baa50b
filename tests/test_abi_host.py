"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every symbol the header
declares, sizes its buffers, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import routed_expert_ffn_wave_amd as ft

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ft_moe.h")

A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails before any use
B = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)    # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(ft_moe_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 22, names
    out = subprocess.run(["nm", "-D", "--defined-only", ft.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(ft_moe_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    assert set(names) == set(ft.EXPORTED)
    for n in names:
        getattr(ft.lib, n)


def test_abi_version():
    assert ft.ft_moe_abi_version() == 1
    m = re.search(r"#define FT_MOE_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == 1


def test_route_proj_validation():
    L = ft.lib
    ws = 16 * 4
    _err(L.ft_moe_route_proj(A, A, 4, 64, 8, 0, B, B, B, B, ws, None), ft.FT_E_INVAL, "k must be")
    _err(L.ft_moe_route_proj(A, A, 4, 64, 513, 2, B, B, B, B, ws, None), ft.FT_E_INVAL, "E must be")
    _err(L.ft_moe_route_proj(A, A, 4, 48, 8, 2, B, B, B, B, ws, None), ft.FT_E_INVAL, "d must be")
    _err(L.ft_moe_route_proj(None, A, 4, 64, 8, 2, B, B, B, B, ws, None), ft.FT_E_INVAL, "x is null")
    _err(L.ft_moe_route_proj(A, A, 4, 64, 8, 2, None, B, B, B, ws, None), ft.FT_E_INVAL, "logits is null")
    _err(L.ft_moe_route_proj(A, A, 4, 64, 8, 2, B, B, B, None, ws, None), ft.FT_E_INVAL, "ws is null")
    _err(L.ft_moe_route_proj(A, A, 40, 64, 8, 2, B, B, B, B, ws, None), ft.FT_E_WORKSPACE, "workspace")
    assert ft.lib.ft_moe_route_proj_workspace(40) == 3 * 16 * 4
    assert L.ft_moe_route_proj(None, None, 0, 64, 8, 2, None, None, None, None, 0, None) == ft.FT_OK


def test_layer_noalloc_refuses_oversize_layers():
    """ft_moe_layer_noalloc refuses a layer whose workspace exceeds its static scratch before any HIP
    call (no GPU needed), and applies ft_moe_layer's own argument checks first."""
    L = ft.lib
    bank = ft.ft_moe_bank(ft.FT_W_FP8_B128, 96, 7168, 2048, 0x10000, 0x20000, 0x30000, 0x40000)
    args = lambda T, k, flags=0: (ctypes.byref(bank), A, -1, A, A, T, 256, k, A, A, A, A, A, A, A, None, A, A, None,  # noqa: E731
                                  flags, None)
    need = L.ft_moe_layer_workspace(ctypes.byref(bank), 4096, 256, 8, -1, 0)
    assert need > ft.FT_NOALLOC_SCRATCH_BYTES
    _err(L.ft_moe_layer_noalloc(*args(4096, 8)), ft.FT_E_WORKSPACE, "static scratch")
    _err(L.ft_moe_layer_noalloc(*args(4, 0)), ft.FT_E_INVAL, "k must be")
    _err(L.ft_moe_layer_noalloc(*args(4, 8, 0x40)), ft.FT_E_INVAL, "unknown flags")


def test_measure_rates_validation():
    """Argument checks of the start-up rate call (before any HIP call)."""
    L = ft.lib
    r = ft.ft_moe_rates()
    big, mib = 64 << 20, 1 << 20
    call = lambda dev=A, nd=big, host=None, nh=0, reps=3, out=ctypes.byref(r): L.ft_moe_measure_rates(  # noqa: E731
        dev, nd, host, nh, reps, out, None)
    _err(call(out=None), ft.FT_E_INVAL, "out is null")
    _err(call(dev=None), ft.FT_E_INVAL, "dev_buf is null")
    _err(call(dev=ctypes.c_void_p(0x10010)), ft.FT_E_INVAL, "256-byte aligned")
    _err(call(nd=big - 1), ft.FT_E_INVAL, "dev_bytes must be at least")
    _err(call(reps=0), ft.FT_E_INVAL, "reps must be")
    _err(call(reps=101), ft.FT_E_INVAL, "reps must be")
    _err(call(host=MIS, nh=mib), ft.FT_E_INVAL, "host_buf is not 16-byte")
    _err(call(host=A, nh=mib - 16), ft.FT_E_INVAL, "host_bytes must be at least")


def test_cache_update_validation():
    L = ft.lib
    args = lambda E, S, ml, q=0.0: (A, E, S, ml, q, A, A, A, A, A, None, A, A)  # noqa: E731
    _err(L.ft_moe_cache_update(*args(0, 4, 1), None), ft.FT_E_INVAL, "E must be")
    _err(L.ft_moe_cache_update(*args(1025, 4, 1), None), ft.FT_E_INVAL, "E must be")
    _err(L.ft_moe_cache_update(*args(8, 0, 0), None), ft.FT_E_INVAL, "n_slots must be")
    _err(L.ft_moe_cache_update(*args(8, 1025, 1), None), ft.FT_E_INVAL, "n_slots must be")
    _err(L.ft_moe_cache_update(*args(8, 4, 5), None), ft.FT_E_INVAL, "max_loads must be")
    _err(L.ft_moe_cache_update(*args(8, 4, -1), None), ft.FT_E_INVAL, "max_loads must be")
    _err(L.ft_moe_cache_update(*args(8, 4, 1, 1.5), None), ft.FT_E_INVAL, "load_fraction must be")
    _err(L.ft_moe_cache_update(*args(8, 4, 1, -0.1), None), ft.FT_E_INVAL, "load_fraction must be")
    _err(L.ft_moe_cache_update(*args(8, 4, 1, float("nan")), None), ft.FT_E_INVAL, "load_fraction must be")
    _err(L.ft_moe_cache_update(None, 8, 4, 1, 0.0, A, A, A, A, A, None, A, A, None), ft.FT_E_INVAL, "counts is null")
    _err(L.ft_moe_cache_update(A, 8, 4, 1, 0.0, A, A, MIS, A, A, None, A, A, None), ft.FT_E_INVAL,
         "last_use is not 16-byte")
    _err(L.ft_moe_cache_update(A, 8, 4, 1, 0.0, A, A, A, A, A, MIS, A, A, None), ft.FT_E_INVAL,
         "load_slot is not 16-byte")
    _err(L.ft_moe_cache_update(A, 8, 4, 1, 0.0, A, A, A, A, A, None, None, A, None), ft.FT_E_INVAL, "loads is null")


def test_cache_fill_validation():
    L = ft.lib
    bank = lambda fmt, n, d, I: ft.ft_moe_bank(fmt, n, d, I, 0x10000, 0x20000, 0x30000, 0x40000)
    src, dst = bank(ft.FT_W_Q4_0, 16, 256, 128), bank(ft.FT_W_Q4_0, 4, 256, 128)
    ref = ctypes.byref
    _err(L.ft_moe_cache_fill(ref(src), ref(bank(ft.FT_W_MXFP4, 4, 256, 128)), A, A, 2, None), ft.FT_E_INVAL,
         "differ in format or shape")
    _err(L.ft_moe_cache_fill(ref(src), ref(bank(ft.FT_W_Q4_0, 4, 256, 192)), A, A, 2, None), ft.FT_E_INVAL,
         "differ in format or shape")
    _err(L.ft_moe_cache_fill(ref(src), ref(dst), A, A, 5, None), ft.FT_E_INVAL, "max_loads must be")
    _err(L.ft_moe_cache_fill(ref(src), ref(dst), None, A, 2, None), ft.FT_E_INVAL, "loads is null")
    _err(L.ft_moe_cache_fill(None, ref(dst), A, A, 2, None), ft.FT_E_INVAL, "bank is null")
    assert L.ft_moe_cache_fill(ref(src), ref(dst), None, None, 0, None) == ft.FT_OK


def test_residual_validation():
    L = ft.lib
    bank = ft.ft_moe_bank(ft.FT_W_Q4_0, 16, 256, 128, 0x10000, 0x20000, 0x30000, 0x40000)
    ref = ctypes.byref(bank)
    _err(L.ft_moe_residual_host(ref, A, A, A, A, None, 4, 16, 0, A, 0), ft.FT_E_INVAL, "k must be")
    _err(L.ft_moe_residual_host(None, A, A, A, A, None, 4, 16, 2, A, 0), ft.FT_E_INVAL, "bank is null")
    _err(L.ft_moe_residual_host(ref, A, A, A, A, None, 4, 16, 2, A, -1), ft.FT_E_INVAL, "n_threads")
    _err(L.ft_moe_residual_host(ref, None, A, A, A, None, 4, 16, 2, A, 0), ft.FT_E_INVAL, "must not be null")
    _err(L.ft_moe_residual_host(ref, A, A, A, A, A, 4, 16, 2, A, 0), ft.FT_E_INVAL, "exactly one of")
    _err(L.ft_moe_residual_host(ref, A, A, A, None, None, 4, 16, 2, A, 0), ft.FT_E_INVAL, "exactly one of")
    assert L.ft_moe_residual_host(ref, None, None, None, None, None, 0, 16, 2, None, 0) == ft.FT_OK
    _err(L.ft_moe_residual_add(A, A, 4, 12, 0, None), ft.FT_E_INVAL, "d must be")
    _err(L.ft_moe_residual_add(A, A, 4, 64, 0x8, None), ft.FT_E_INVAL, "unknown flags")
    _err(L.ft_moe_residual_add(None, A, 4, 64, 0, None), ft.FT_E_INVAL, "out is null")
    assert L.ft_moe_residual_add(None, None, 0, 64, 0, None) == ft.FT_OK


def test_residual_host_bf16_on_cpu():
    """The host residual needs no GPU: a bf16 bank laid out by hand in the documented device layout
    (16-byte chunks interleaved in 64-row blocks; W13 device block b = gate rows 32b.. then up rows)
    against the fp32 oracle's FFN of the same weights, rounded as the device rounds h and y."""
    import numpy as np
    import torch
    import oracle
    from host_banks import bf16_bank
    rng = np.random.default_rng(5)
    T, d, E, k, I = 5, 128, 3, 2, 64
    hb, w13, w2 = bf16_bank(rng, E, d, I)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    ids = torch.tensor([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0]], dtype=torch.int32)
    wts = torch.from_numpy(rng.random((T, k)).astype(np.float32))
    mask = torch.tensor([0b01, 0b11, 0b00, 0b10, 0b01], dtype=torch.int32)
    got = ft.ft_moe_residual_host(hb, x, ids, wts, mask, n_threads=3).numpy()
    xf = x.float().numpy()
    ref = np.zeros((T, d), np.float64)
    for t in range(T):
        for j in range(k):
            if (int(mask[t]) >> j) & 1:
                e = int(ids[t, j])
                _, y = oracle.swiglu_ffn(xf[t:t + 1], w13[e], w2[e])
                ref[t] += float(wts[t, j]) * y[0].astype(np.float64)
    assert np.array_equal(got[2], np.zeros(d, np.float32))
    # the slot-table form: experts 0 and 2 cold for the tokens whose mask marks them
    slots = torch.tensor([-1, 5, -1], dtype=torch.int32)
    by_slots = ft.ft_moe_residual_host(hb, x, ids, wts, None, n_threads=2, slot_of_expert=slots).numpy()
    mask2 = torch.tensor([sum(1 << j for j in range(k) if int(slots[int(ids[t, j])]) < 0) for t in range(T)],
                         dtype=torch.int32)
    assert np.array_equal(by_slots, ft.ft_moe_residual_host(hb, x, ids, wts, mask2, n_threads=2).numpy())
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 5e-3, rel


def test_moelayer_takes_bf16_output_from_flags():
    """FT_OUT_BF16 given in `flags` makes the layer's own output buffer bf16 (as out_bf16=True does):
    the layer call would otherwise write bf16 values into an fp32 buffer."""
    import torch
    bank = ft.DeviceBank.empty(ft.FT_W_Q4_0, 4, 256, 128, device="cpu")
    slots = torch.arange(4, dtype=torch.int32)
    a = ft.MoELayer(bank, slots, 2, 8, flags=ft.FT_OUT_BF16)
    b = ft.MoELayer(bank, slots, 2, 8, out_bf16=True)
    assert a.out.dtype == b.out.dtype == torch.bfloat16
    assert a.flags == b.flags and a.out_flags == b.out_flags == ft.FT_OUT_BF16


def test_residual_host_fp8_on_cpu():
    """The FP8-B128 decode of the host residual (the vector path where the host has AVX-512): a bank
    whose codes cover every finite e4m3 byte, laid out by hand in the documented device layout (16
    codes per chunk, 64-row interleave, fp32 scales per 128 x 128 block of logical rows), against the
    oracle's FFN of the weights its own e4m3 decoder gives."""
    import numpy as np
    import torch
    import oracle
    from host_banks import fp8_bank
    rng = np.random.default_rng(6)
    T, d, E, k, I = 3, 256, 2, 2, 128
    table = np.array([oracle.e4m3_value(int(c)) for c in range(256)], np.float32)
    hb, v13, v2 = fp8_bank(rng, E, d, I, table)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    ids = torch.tensor([[0, 1], [1, 0], [0, 1]], dtype=torch.int32)
    wts = torch.tensor([[0.6, 0.4], [0.7, 0.3], [0.5, 0.5]], dtype=torch.float32)
    mask = torch.tensor([0b11, 0b01, 0b10], dtype=torch.int32)
    got = ft.ft_moe_residual_host(hb, x, ids, wts, mask, n_threads=2).numpy()
    xf = x.float().numpy()
    ref = np.zeros((T, d), np.float64)
    for t in range(T):
        for j in range(k):
            if (int(mask[t]) >> j) & 1:
                e = int(ids[t, j])
                _, y = oracle.swiglu_ffn(xf[t:t + 1], v13[e], v2[e])
                ref[t] += float(wts[t, j]) * y[0].astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert np.isfinite(got).all() and rel < 5e-3, rel


def _err(rc, code, pattern):
    assert rc == code, (rc, ft.ft_moe_last_error())
    assert re.search(pattern, ft.ft_moe_last_error()), ft.ft_moe_last_error()


def test_route_validation():
    L = ft.lib
    _err(L.ft_moe_route(A, 4, 8, 0, B, B, None), ft.FT_E_INVAL, "k must be")
    _err(L.ft_moe_route(A, 4, 8, 9, B, B, None), ft.FT_E_INVAL, "k must be")
    _err(L.ft_moe_route(A, 4, 64, 33, B, B, None), ft.FT_E_INVAL, "k must be")
    _err(L.ft_moe_route(A, 4, 0, 1, B, B, None), ft.FT_E_INVAL, "E must be")
    _err(L.ft_moe_route(A, 4, 1025, 1, B, B, None), ft.FT_E_INVAL, "E must be")
    _err(L.ft_moe_route(A, -1, 8, 2, B, B, None), ft.FT_E_INVAL, "T must be")
    _err(L.ft_moe_route(None, 4, 8, 2, B, B, None), ft.FT_E_INVAL, "logits is null")
    _err(L.ft_moe_route(A, 4, 8, 2, None, B, None), ft.FT_E_INVAL, "ids is null")
    _err(L.ft_moe_route(MIS, 4, 8, 2, B, B, None), ft.FT_E_INVAL, "logits is not 16-byte aligned")
    # T == 0 is a no-op that succeeds without touching any pointer
    assert L.ft_moe_route(None, 0, 8, 2, None, None, None) == ft.FT_OK
    assert ft.ft_moe_last_error() == ""


def test_permute_validation_and_workspace():
    L = ft.lib
    assert L.ft_moe_permute_workspace(8, 128, 8) == 0           # single-block path
    assert L.ft_moe_permute_workspace(2048, 128, 8) == 0        # 16384 entries: still one block
    assert L.ft_moe_permute_workspace(4096, 128, 8) == 32 * 128 * 4
    assert L.ft_moe_permute_workspace(8192, 128, 8) == 64 * 128 * 4
    assert L.ft_moe_permute_workspace(16384, 256, 8) == 128 * 256 * 4
    _err(L.ft_moe_permute(A, 8192, 128, 8, B, B, B, B, None, 0, None), ft.FT_E_WORKSPACE, "needs 32768 bytes")
    _err(L.ft_moe_permute(A, 8192, 128, 8, B, B, B, B, A, 100, None), ft.FT_E_WORKSPACE, "needs")
    _err(L.ft_moe_permute(A, 8192, 128, 8, B, B, B, B, MIS, 1 << 20, None), ft.FT_E_INVAL, "ws is not")
    _err(L.ft_moe_permute(A, 4, 8, 2, None, B, B, B, None, 0, None), ft.FT_E_INVAL, "counts is null")
    _err(L.ft_moe_permute(None, 4, 8, 2, B, B, B, B, None, 0, None), ft.FT_E_INVAL, "ids is null")
    _err(L.ft_moe_permute(A, 4, 8, 2, B, B, MIS, B, None, 0, None), ft.FT_E_INVAL, "gather is not")


def _bank(fmt=ft.FT_W_Q4_0, n=8, d=256, I=512, s=True):
    return ft.ft_moe_bank(fmt, n, d, I, A.value, B.value, A.value if s else None, B.value if s else None)


def test_bank_bytes():
    L = ft.lib
    d, I, n = 2048, 768, 128
    assert L.ft_moe_bank_bytes(ft.FT_W_BF16, n, d, I, 0) == n * 2 * I * d * 2
    assert L.ft_moe_bank_bytes(ft.FT_W_BF16, n, d, I, 2) == 0
    assert L.ft_moe_bank_bytes(ft.FT_W_Q4_0, n, d, I, 0) == n * 2 * I * d // 2
    assert L.ft_moe_bank_bytes(ft.FT_W_Q4_0, n, d, I, 3) == n * d * (I // 32) * 2
    assert L.ft_moe_bank_bytes(ft.FT_W_MXFP4, n, d, I, 2) == n * 2 * I * (d // 32)
    assert L.ft_moe_bank_bytes(ft.FT_W_FP8_B128, 96, 7168, 2048, 2) == 96 * 32 * 56 * 4
    assert L.ft_moe_bank_bytes(ft.FT_W_FP8_B128, 96, 7168, 2000, 0) == 0     # I not a multiple of 128
    assert L.ft_moe_bank_bytes(7, 1, 256, 256, 0) == 0
    # NVFP4: codes as MXFP4; two e4m3 bytes per (row, chunk), then one fp32 matrix scale per slot
    assert L.ft_moe_bank_bytes(ft.FT_W_NVFP4, n, d, I, 0) == n * 2 * I * d // 2
    assert L.ft_moe_bank_bytes(ft.FT_W_NVFP4, n, d, I, 2) == n * 2 * I * (d // 32) * 2 + n * 4
    assert L.ft_moe_bank_bytes(ft.FT_W_NVFP4, n, d, I, 3) == n * d * (I // 32) * 2 + n * 4
    # per-weight cost of each format: 2, 18/32, 17/32, 1 + 4/16384, 9/16 (+ two fp32 per slot) bytes
    for fmt, bpw, extra in ((0, 2.0, 0), (1, 18 / 32, 0), (2, 17 / 32, 0), (3, 1 + 4 / 16384, 0), (4, 9 / 16, 8)):
        tot = sum(L.ft_moe_bank_bytes(fmt, 1, 7168, 2048, w) for w in range(4))
        assert tot - extra == pytest.approx(3 * 7168 * 2048 * bpw, rel=1e-12)


def test_grouped_ffn_validation():
    L = ft.lib
    b = _bank()
    ws = 1 << 20
    call = lambda **kw: L.ft_moe_grouped_ffn(
        kw.get("bank", ctypes.byref(b)), kw.get("slot", A), kw.get("shared", -1), kw.get("x", A), kw.get("T", 16),
        kw.get("E", 8), kw.get("k", 2), kw.get("off", A), kw.get("gather", A), kw.get("y", A), kw.get("ysh", None),
        kw.get("ws", A), kw.get("ws_bytes", ws), kw.get("flags", 0), None)
    _err(call(bank=None), ft.FT_E_INVAL, "bank is null")
    _err(call(ws_bytes=10), ft.FT_E_WORKSPACE, "needs")
    _err(call(ws=None), ft.FT_E_WORKSPACE, "null pointer")
    _err(call(flags=3), ft.FT_E_INVAL, "exclusive")
    _err(call(flags=8), ft.FT_E_INVAL, "unknown flags")
    _err(call(shared=8), ft.FT_E_INVAL, "shared_slot")
    _err(call(shared=3), ft.FT_E_INVAL, "y_shared")
    _err(call(ysh=B), ft.FT_E_INVAL, "y_shared")
    _err(call(x=None), ft.FT_E_INVAL, "x is null")
    _err(call(x=MIS), ft.FT_E_INVAL, "x is not 16-byte aligned")
    _err(call(k=3, E=2), ft.FT_E_INVAL, "k must be")
    nob = _bank(s=False)
    _err(call(bank=ctypes.byref(nob)), ft.FT_E_INVAL, "scale arrays")
    bad = _bank(fmt=9)
    _err(call(bank=ctypes.byref(bad)), ft.FT_E_UNSUPPORTED, "unknown weight format")
    odd = _bank(d=192)
    _err(call(bank=ctypes.byref(odd)), ft.FT_E_INVAL, "multiple of 128")
    odd_i = _bank(d=256, I=96)
    _err(call(bank=ctypes.byref(odd_i)), ft.FT_E_INVAL, "multiple of 64")
    fp8 = _bank(fmt=ft.FT_W_FP8_B128, d=256, I=64)
    _err(call(bank=ctypes.byref(fp8)), ft.FT_E_INVAL, "FP8_B128 needs I")
    # workspace query: the work-queue counters, then bf16 h rows for every routed pair (and the shared expert)
    assert L.ft_moe_grouped_ffn_workspace(ctypes.byref(b), 16, 8, 2, -1, 0) == 4 * 8 * 16 * 4 + 16 * 2 * 512 * 2
    assert L.ft_moe_grouped_ffn_workspace(ctypes.byref(b), 16, 8, 2, 3, 0) == 4 * 8 * 16 * 4 + (16 * 2 + 16) * 512 * 2
    assert call(T=0) == ft.FT_OK


def test_grouped_ffn_workspace_holds_activation_terms():
    """MXFP4 and FP8-B128 banks whose shapes the scaled-MFMA kernels take add the two-term activations
    of x (T rows of d) and of every h row (of I) to the grouped FFN's workspace, unless
    FT_GEMM_WIDEN sends their groups to the bf16 kernels; other formats need the h rows only."""
    L = ft.lib
    T, E, k, d, I = 300, 16, 4, 512, 256
    h = T * k * I * 2
    r256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    q = 4 * 8 * 16 * 4   # the work-queue counters of the call's four kernel launches
    for fmt, cb in ((ft.FT_W_MXFP4, 48), (ft.FT_W_FP8_B128, 64)):
        b = _bank(fmt=fmt, n=E, d=d, I=I)
        terms = lambda rows, K: r256(rows * (K // 32) * cb) + r256(rows * (K // 32) * 2)  # noqa: E731
        full = L.ft_moe_grouped_ffn_workspace(ctypes.byref(b), T, E, k, -1, 0)
        assert full == q + r256(h) + terms(T, d) + terms(T * k, I), (fmt, full)
        assert L.ft_moe_grouped_ffn_workspace(ctypes.byref(b), T, E, k, -1, ft.FT_GEMM_WIDEN) == q + r256(h)
    b = _bank(fmt=ft.FT_W_BF16, n=E, d=d, I=I)
    assert L.ft_moe_grouped_ffn_workspace(ctypes.byref(b), T, E, k, -1, 0) == q + r256(h)


def test_layer_validation_and_workspace():
    L = ft.lib
    b = _bank(fmt=ft.FT_W_Q4_0, n=8, d=256, I=512)
    ws = 1 << 22

    def call(**kw):
        return L.ft_moe_layer(kw.get("bank", ctypes.byref(b)), kw.get("slot", A), kw.get("shared", -1),
                              kw.get("logits", A), kw.get("x", A), kw.get("T", 8), kw.get("E", 8), kw.get("k", 2),
                              kw.get("ids", A), kw.get("w", A), kw.get("counts", A), kw.get("offsets", A),
                              kw.get("gather", A), kw.get("inv", A), kw.get("y", A), kw.get("ysh", None),
                              kw.get("out", B), kw.get("mask", None), kw.get("ws", A), kw.get("ws_bytes", ws),
                              kw.get("flags", 0), None)
    _err(call(bank=None), ft.FT_E_INVAL, "bank is null")
    _err(call(flags=0x40), ft.FT_E_INVAL, "unknown flags")
    _err(call(flags=3), ft.FT_E_INVAL, "exclusive")
    _err(call(k=9), ft.FT_E_INVAL, "k must be")
    _err(call(shared=3), ft.FT_E_INVAL, "y_shared")
    _err(call(ws_bytes=100), ft.FT_E_WORKSPACE, "needs")
    _err(call(ws=MIS), ft.FT_E_INVAL, "ws is not")
    _err(call(logits=None), ft.FT_E_INVAL, "logits is null")
    _err(call(out=MIS), ft.FT_E_INVAL, "out is not 16-byte aligned")
    _err(call(inv=None), ft.FT_E_INVAL, "inv is null")
    _err(call(counts=None), ft.FT_E_INVAL, "counts is null")
    # workspace: control words, fused counters and h rows for decode sizes; h rows and the
    # permutation's workspace otherwise
    fused = L.ft_moe_layer_workspace(ctypes.byref(b), 8, 8, 2, -1, 0)
    unfused = L.ft_moe_layer_workspace(ctypes.byref(b), 8, 8, 2, -1, ft.FT_LAYER_UNFUSED)
    h = 8 * 2 * 512 * 2
    ctl = 10 * 64 * 4   # status word, a work-queue counter per XCD and the exit counter, each on its own line
    rproj = lambda T: -(-((T + 15) // 16 * 64) // 256) * 256  # noqa: E731  (router-projection counters, 256-aligned)
    qctr = 4 * 8 * 16 * 4  # the four calls' work-queue counters (grouped FFN kernels)
    assert unfused == ctl + rproj(8) + qctr + h
    assert fused > unfused
    big = L.ft_moe_layer_workspace(ctypes.byref(b), 4096, 8, 2, -1, 0)
    assert big == ctl + rproj(4096) + qctr + 4096 * 2 * 512 * 2
    assert L.ft_moe_layer_workspace(ctypes.byref(b), 16, 8, 9, -1, 0) == 0
    assert L.ft_moe_layer_workspace(None, 16, 8, 2, -1, 0) == 0


def test_layer_proj_validation():
    """ft_moe_layer_proj's own checks, then those of ft_moe_layer (before any HIP call)."""
    L = ft.lib
    b = _bank(fmt=ft.FT_W_Q4_0, n=8, d=256, I=512)
    call = lambda wr=A, lg=B, E=8, T=4, k=2, flags=0: L.ft_moe_layer_proj(  # noqa: E731
        ctypes.byref(b), A, -1, A, wr, T, E, k, lg, A, A, A, A, A, A, A, None, A, None, A, 1 << 24, flags, None)
    _err(call(E=513, k=2), ft.FT_E_INVAL, "E must be at most 512")
    _err(call(wr=None), ft.FT_E_INVAL, "w_router is null")
    _err(call(lg=None), ft.FT_E_INVAL, "logits is null")
    _err(call(k=9), ft.FT_E_INVAL, "k must be")
    _err(call(flags=0x40), ft.FT_E_INVAL, "unknown flags")


def test_combine_validation():
    L = ft.lib
    call = lambda **kw: L.ft_moe_combine(kw.get("y", A), kw.get("ysh", None), kw.get("ids", A), kw.get("w", A),
                                         kw.get("inv", A), kw.get("slot", A), kw.get("T", 4), kw.get("E", 8),
                                         kw.get("k", 2), kw.get("d", 256), kw.get("out", B), kw.get("mask", None),
                                         kw.get("flags", 0), None)
    _err(call(d=250), ft.FT_E_INVAL, "multiple of 8")
    _err(call(flags=1), ft.FT_E_INVAL, "unknown flags")
    _err(call(out=None), ft.FT_E_INVAL, "out is null")
    _err(call(mask=MIS), ft.FT_E_INVAL, "residual_mask is not")
    _err(call(inv=None), ft.FT_E_INVAL, "inv is null")
    assert call(T=0) == ft.FT_OK


def test_pack_and_dequant_validation():
    L = ft.lib
    b = _bank(fmt=ft.FT_W_Q4_0, n=2, d=256, I=256)
    _err(L.ft_moe_pack_bank(1, 2, 256, 512, A, B, None, None, ctypes.byref(b), None), ft.FT_E_INVAL, "does not match")
    _err(L.ft_moe_pack_bank(1, 2, 256, 256, None, B, None, None, ctypes.byref(b), None), ft.FT_E_INVAL, "null")
    _err(L.ft_moe_pack_bank(1, 2, 256, 256, ctypes.c_void_p(0x10001), B, None, None, ctypes.byref(b), None),
         ft.FT_E_INVAL, "2-byte aligned")
    _err(L.ft_moe_dequant(ctypes.byref(b), 2, 0, A, None), ft.FT_E_INVAL, "slot 2 out of range")
    _err(L.ft_moe_dequant(ctypes.byref(b), 0, 2, A, None), ft.FT_E_INVAL, "which must be")
    _err(L.ft_moe_dequant(ctypes.byref(b), 0, 0, None, None), ft.FT_E_INVAL, "out is null")


def test_binding_has_no_oracle_dependency():
    """The product path must not import the oracle or the input generator."""
    import sys
    pkg = os.path.join(ROOT, "routed_expert_ffn_wave_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\b(import|from)\s+(oracle|synth)\b", src), f
                assert "ftoracle" not in src, f
    assert "oracle" not in {m.split(".")[0] for m in sys.modules if m.startswith("routed_expert")}
