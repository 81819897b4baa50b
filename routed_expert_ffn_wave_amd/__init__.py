"""Python binding of libftmoe.so, the gfx950 HIP library of one Mixture-of-Experts layer.

The functions below carry the C ABI's names (include/ft_moe.h) and only marshal arguments: torch
tensors provide device memory and the current torch stream provides the HIP stream; every step of
the layer runs in the library's HIP kernels.  Importing this package fails if the library has not
been built (python -m routed_expert_ffn_wave_amd.build); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libftmoe.so")

FT_OK, FT_E_INVAL, FT_E_UNSUPPORTED, FT_E_WORKSPACE, FT_E_HIP, FT_E_INTERNAL = range(6)
FT_W_BF16, FT_W_Q4_0, FT_W_MXFP4, FT_W_FP8_B128, FT_W_NVFP4 = range(5)
FT_PATH_AUTO, FT_PATH_GEMV, FT_PATH_GEMM = 0, 1, 2
FT_OUT_BF16 = 4
FT_LAYER_UNFUSED = 8
FT_GEMM_WIDEN = 16   # MXFP4 / FP8-B128 GEMM groups on the bf16 MFMA (weights widened) instead of fp4 / fp8
FT_PATH_MASK = 3
LAYER_MAX_T = 16   # largest T of the fused decode kernels
FT_NOALLOC_SCRATCH_BYTES = 8 << 20   # static scratch of ft_moe_layer_noalloc, per device

STATUS_NAMES = {0: "FT_OK", 1: "FT_E_INVAL", 2: "FT_E_UNSUPPORTED", 3: "FT_E_WORKSPACE", 4: "FT_E_HIP",
                5: "FT_E_INTERNAL"}


class FtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class ft_moe_bank(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("d", ctypes.c_int32),
                ("I", ctypes.c_int32), ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("s13", ctypes.c_void_p), ("s2", ctypes.c_void_p)]


class ft_moe_rates(ctypes.Structure):
    _fields_ = [("hbm_read_gbs", ctypes.c_double), ("host_read_gbs", ctypes.c_double),
                ("mfma_bf16_tflops", ctypes.c_double), ("mfma_fp8_tflops", ctypes.c_double),
                ("mfma_fp6_fp4_tflops", ctypes.c_double), ("mfma_clock_ghz", ctypes.c_double),
                ("compute_units", ctypes.c_int32), ("stream_blocks", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m routed_expert_ffn_wave_amd.build`")
    # torch is imported first so that the library binds to the HIP runtime torch already loaded
    lib = ctypes.CDLL(LIB_PATH)
    P, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    BP = ctypes.POINTER(ft_moe_bank)
    sig = {
        "ft_moe_abi_version": ([], i),
        "ft_moe_last_error": ([], ctypes.c_char_p),
        "ft_moe_route": ([P, i, i, i, P, P, P], i),
        "ft_moe_route_proj_workspace": ([i], sz),
        "ft_moe_route_proj": ([P, P, i, i, i, i, P, P, P, P, sz, P], i),
        "ft_moe_permute_workspace": ([i, i, i], sz),
        "ft_moe_permute": ([P, i, i, i, P, P, P, P, P, sz, P], i),
        "ft_moe_grouped_ffn_workspace": ([BP, i, i, i, i, i], sz),
        "ft_moe_grouped_ffn": ([BP, P, i, P, i, i, i, P, P, P, P, P, sz, i, P], i),
        "ft_moe_combine": ([P, P, P, P, P, P, i, i, i, i, P, P, i, P], i),
        "ft_moe_bank_bytes": ([i, i, i, i, i], sz),
        "ft_moe_pack_bank": ([i, i, i, i, P, P, P, P, BP, P], i),
        "ft_moe_dequant": ([BP, i, i, P, P], i),
        "ft_moe_layer_workspace": ([BP, i, i, i, i, i], sz),
        "ft_moe_layer": ([BP, P, i, P, P, i, i, i, P, P, P, P, P, P, P, P, P, P, P, sz, i, P], i),
        "ft_moe_layer_noalloc": ([BP, P, i, P, P, i, i, i, P, P, P, P, P, P, P, P, P, P, P, i, P], i),
        "ft_moe_layer_proj": ([BP, P, i, P, P, i, i, i, P, P, P, P, P, P, P, P, P, P, P, P, sz, i, P], i),
        "ft_moe_cache_update": ([P, i, i, i, ctypes.c_float, P, P, P, P, P, P, P, P, P], i),
        "ft_moe_cache_fill": ([BP, BP, P, P, i, P], i),
        "ft_moe_residual_host": ([BP, P, P, P, P, P, i, i, i, P, i], i),
        "ft_moe_residual_add": ([P, P, i, i, i, P], i),
        "ft_moe_measure_rates": ([P, sz, P, sz, i, ctypes.POINTER(ft_moe_rates), P], i),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()

EXPORTED = ("ft_moe_abi_version", "ft_moe_last_error", "ft_moe_route", "ft_moe_route_proj_workspace",
            "ft_moe_route_proj", "ft_moe_permute_workspace",
            "ft_moe_permute", "ft_moe_grouped_ffn_workspace", "ft_moe_grouped_ffn", "ft_moe_combine",
            "ft_moe_bank_bytes", "ft_moe_pack_bank", "ft_moe_dequant", "ft_moe_layer_workspace", "ft_moe_layer",
            "ft_moe_layer_noalloc", "ft_moe_cache_update", "ft_moe_cache_fill", "ft_moe_residual_host", "ft_moe_residual_add",
            "ft_moe_measure_rates", "ft_moe_layer_proj")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc: int):
    if rc != FT_OK:
        raise FtError(rc, lib.ft_moe_last_error().decode())


def ft_moe_abi_version() -> int:
    return lib.ft_moe_abi_version()


def ft_moe_last_error() -> str:
    return lib.ft_moe_last_error().decode()


# ------------------------------------------------------------------------------------- banks

class DeviceBank:
    """Device-layout expert bank: torch tensors that own the arrays, plus the C description."""

    def __init__(self, fmt: int, n_slots: int, d: int, I: int, w13, w2, s13=None, s2=None):
        self.fmt, self.n_slots, self.d, self.I = fmt, n_slots, d, I
        self.w13, self.w2, self.s13, self.s2 = w13, w2, s13, s2
        self.desc = ft_moe_bank(fmt, n_slots, d, I, w13.data_ptr(), w2.data_ptr(),
                                None if s13 is None else s13.data_ptr(), None if s2 is None else s2.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self.desc)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.w13, self.w2, self.s13, self.s2) if t is not None)

    @staticmethod
    def empty(fmt: int, n_slots: int, d: int, I: int, device="cuda") -> "DeviceBank":
        arrs = []
        for which in range(4):
            n = lib.ft_moe_bank_bytes(fmt, n_slots, d, I, which)
            if n == 0 and which < 2:
                raise FtError(FT_E_INVAL, f"invalid bank shape fmt={fmt} n_slots={n_slots} d={d} I={I}")
            arrs.append(torch.empty(n, dtype=torch.uint8, device=device) if n else None)
        return DeviceBank(fmt, n_slots, d, I, *arrs)

    def to_pinned_host(self) -> "DeviceBank":
        """The same bank copied into pinned host memory (the cold tier ft_moe_cache_fill reads)."""
        arrs = []
        for t in (self.w13, self.w2, self.s13, self.s2):
            if t is None:
                arrs.append(None)
                continue
            h = torch.empty(t.numel(), dtype=torch.uint8, pin_memory=True)
            h.copy_(t.view(torch.uint8).reshape(-1))
            arrs.append(h)
        return DeviceBank(self.fmt, self.n_slots, self.d, self.I, *arrs)


def ft_moe_bank_bytes(fmt: int, n_slots: int, d: int, I: int, which: int) -> int:
    return lib.ft_moe_bank_bytes(fmt, n_slots, d, I, which)


def ft_moe_pack_bank(fmt: int, n_slots: int, d: int, I: int, canon_w13, canon_w2, canon_s13=None, canon_s2=None,
                     dst: DeviceBank | None = None, stream=None) -> DeviceBank:
    dst = DeviceBank.empty(fmt, n_slots, d, I, device=canon_w13.device) if dst is None else dst
    _check(lib.ft_moe_pack_bank(fmt, n_slots, d, I, _ptr(canon_w13), _ptr(canon_w2), _ptr(canon_s13),
                                _ptr(canon_s2), dst.ref, _stream(stream)))
    return dst


def ft_moe_dequant(bank: DeviceBank, slot: int, which: int, out=None, stream=None) -> torch.Tensor:
    rows, K = (2 * bank.I, bank.d) if which == 0 else (bank.d, bank.I)
    out = torch.empty(rows, K, dtype=torch.float32, device=bank.w13.device) if out is None else out
    _check(lib.ft_moe_dequant(bank.ref, slot, which, _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------------------------------------- expert cache

def ft_moe_cache_update(counts, slot_of_expert, expert_of_slot, last_use, tick, max_loads: int,
                        load_fraction: float = 0.0, compute_slot=None, load_slot=None, loads=None, n_loads=None,
                        stream=None):
    """One step of the global LRU expert cache on device-resident state (int32 tensors; last_use and
    tick hold uint32 bits).  Returns (compute_slot [E], loads [max_loads][2], n_loads [1]); load_slot
    [E] is written when given."""
    E, S = counts.shape[0], expert_of_slot.shape[0]
    dev = counts.device
    compute_slot = torch.empty(E, dtype=torch.int32, device=dev) if compute_slot is None else compute_slot
    loads = torch.empty(max(max_loads, 1), 2, dtype=torch.int32, device=dev) if loads is None else loads
    n_loads = torch.empty(1, dtype=torch.int32, device=dev) if n_loads is None else n_loads
    _check(lib.ft_moe_cache_update(_ptr(counts), E, S, max_loads, float(load_fraction), _ptr(slot_of_expert),
                                   _ptr(expert_of_slot), _ptr(last_use), _ptr(tick), _ptr(compute_slot),
                                   _ptr(load_slot), _ptr(loads), _ptr(n_loads), _stream(stream)))
    return compute_slot, loads, n_loads


def ft_moe_cache_fill(src: DeviceBank, dst: DeviceBank, loads, n_loads, max_loads: int, stream=None):
    """Copy the listed experts from `src` (every expert, pinned host or device memory) into `dst`."""
    _check(lib.ft_moe_cache_fill(src.ref, dst.ref, _ptr(loads), _ptr(n_loads), max_loads, _stream(stream)))


class ExpertCache:
    """Device state of the global LRU expert cache over slots 0..n_slots-1 of a device bank, and the
    buffers one step writes.  Starts with every slot empty."""

    def __init__(self, E: int, n_slots: int, max_loads: int, device="cuda", load_fraction: float = 0.0):
        self.E, self.n_slots, self.max_loads, self.load_fraction = E, n_slots, max_loads, load_fraction
        self.slot_of_expert = torch.full((E,), -1, dtype=torch.int32, device=device)
        self.expert_of_slot = torch.full((n_slots,), -1, dtype=torch.int32, device=device)
        self.last_use = torch.zeros(n_slots, dtype=torch.int32, device=device)
        self.tick = torch.zeros(1, dtype=torch.int32, device=device)
        self.compute_slot = torch.empty(E, dtype=torch.int32, device=device)
        self.load_slot = torch.empty(E, dtype=torch.int32, device=device)
        self.loads = torch.empty(max(max_loads, 1), 2, dtype=torch.int32, device=device)
        self.n_loads = torch.zeros(1, dtype=torch.int32, device=device)

    def update(self, counts, stream=None):
        return ft_moe_cache_update(counts, self.slot_of_expert, self.expert_of_slot, self.last_use, self.tick,
                                   self.max_loads, self.load_fraction, self.compute_slot, self.load_slot, self.loads,
                                   self.n_loads, stream)

    def fill(self, src: DeviceBank, dst: DeviceBank, stream=None):
        ft_moe_cache_fill(src, dst, self.loads, self.n_loads, self.max_loads, stream)


# ------------------------------------------------------------------------------------- cold-expert residual

def ft_moe_residual_host(host_bank: DeviceBank, x, ids, w, residual_mask=None, out=None, n_threads: int = 0,
                         E: int | None = None, slot_of_expert=None):
    """Host compute of the cold pairs (residual_mask bits, or slot_of_expert < 0 when the mask is not
    given): all arguments host (CPU) tensors; host_bank holds every expert (expert e in slot e) in host
    memory; E defaults to its slot count.  Returns out fp32 [T][d]."""
    T, k = ids.shape
    d = x.shape[1]
    out = torch.empty(T, d, dtype=torch.float32) if out is None else out
    E = int(host_bank.n_slots) if E is None else E
    _check(lib.ft_moe_residual_host(host_bank.ref, _ptr(x), _ptr(ids), _ptr(w), _ptr(residual_mask),
                                    _ptr(slot_of_expert), T, E, k, _ptr(out), n_threads))
    return out


def ft_moe_residual_add(out, residual, flags: int = 0, stream=None):
    """out += residual on the device (out fp32, or bf16 with FT_OUT_BF16)."""
    T, d = residual.shape
    _check(lib.ft_moe_residual_add(_ptr(out), _ptr(residual), T, d, flags, _stream(stream)))
    return out


def ft_moe_measure_rates(dev_bytes: int = 1 << 30, host_bytes: int = 256 << 20, reps: int = 3, stream=None) -> dict:
    """The device's rates (ft_moe_measure_rates): a device buffer of dev_bytes and a pinned host buffer
    of host_bytes (0: no host link figure) are allocated here for the call.  Blocks until measured."""
    dev = torch.empty(dev_bytes, dtype=torch.uint8, device="cuda")
    host = torch.ones(host_bytes, dtype=torch.uint8, pin_memory=True) if host_bytes else None
    r = ft_moe_rates()
    _check(lib.ft_moe_measure_rates(_ptr(dev), dev_bytes, _ptr(host), host_bytes if host is not None else 0, reps,
                                    ctypes.byref(r), _stream(stream)))
    return {name: getattr(r, name) for name, _ in ft_moe_rates._fields_}


# ------------------------------------------------------------------------------------- the four calls

def ft_moe_route(logits: torch.Tensor, k: int, ids=None, w=None, stream=None):
    T, E = logits.shape
    ids = torch.empty(T, k, dtype=torch.int32, device=logits.device) if ids is None else ids
    w = torch.empty(T, k, dtype=torch.float32, device=logits.device) if w is None else w
    _check(lib.ft_moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def ft_moe_route_proj_workspace(T: int) -> int:
    return lib.ft_moe_route_proj_workspace(T)


def ft_moe_route_proj(x: torch.Tensor, w_router: torch.Tensor, k: int, logits=None, ids=None, w=None, ws=None,
                      stream=None):
    """Router logits x . w_router^T (bf16 [T][d] and [E][d]) and their top-k, in one launch.
    `ws`: a zero-filled workspace of ft_moe_route_proj_workspace(T) bytes (allocated zeroed when
    not given); the call leaves it zero."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty(T, E, dtype=torch.float32, device=dev) if logits is None else logits
    ids = torch.empty(T, k, dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty(T, k, dtype=torch.float32, device=dev) if w is None else w
    need = lib.ft_moe_route_proj_workspace(T)
    if ws is None:
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev)
    _check(lib.ft_moe_route_proj(_ptr(x), _ptr(w_router), T, d, E, k, _ptr(logits), _ptr(ids), _ptr(w), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)))
    return logits, ids, w


def ft_moe_permute_workspace(T: int, E: int, k: int) -> int:
    return lib.ft_moe_permute_workspace(T, E, k)


def ft_moe_permute(ids: torch.Tensor, E: int, counts=None, offsets=None, gather=None, inv=None, ws=None, stream=None):
    T, k = ids.shape
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    gather = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev) if gather is None else gather
    inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev) if inv is None else inv
    need = lib.ft_moe_permute_workspace(T, E, k)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.ft_moe_permute(_ptr(ids), T, E, k, _ptr(counts), _ptr(offsets), _ptr(gather), _ptr(inv), _ptr(ws),
                              ws_bytes, _stream(stream)))
    return counts, offsets, gather[: T * k], inv[: T * k]


def ft_moe_grouped_ffn_workspace(bank: DeviceBank, T: int, E: int, k: int, shared_slot: int = -1, flags: int = 0) -> int:
    return lib.ft_moe_grouped_ffn_workspace(bank.ref, T, E, k, shared_slot, flags)


def ft_moe_grouped_ffn(bank: DeviceBank, slot_of_expert, x, k: int, offsets, gather, shared_slot: int = -1,
                       y_sorted=None, y_shared=None, ws=None, flags: int = FT_PATH_AUTO, stream=None):
    T, d = x.shape
    E = slot_of_expert.shape[0]
    dev = x.device
    y_sorted = torch.empty(max(T * k, 1), d, dtype=torch.bfloat16, device=dev) if y_sorted is None else y_sorted
    if shared_slot >= 0 and y_shared is None:
        y_shared = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    need = lib.ft_moe_grouped_ffn_workspace(bank.ref, T, E, k, shared_slot, flags)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib.ft_moe_grouped_ffn(bank.ref, _ptr(slot_of_expert), shared_slot, _ptr(x), T, E, k, _ptr(offsets),
                                  _ptr(gather), _ptr(y_sorted), _ptr(y_shared if shared_slot >= 0 else None),
                                  _ptr(ws), ws.numel() * ws.element_size(), flags, _stream(stream)))
    return y_sorted[: T * k], (y_shared if shared_slot >= 0 else None)


def ft_moe_combine(y_sorted, y_shared, ids, w, inv, slot_of_expert, d: int, out=None, residual_mask=None,
                   flags: int = 0, want_mask: bool = True, stream=None):
    T, k = ids.shape
    E = slot_of_expert.shape[0]
    dev = ids.device
    if out is None:
        out = torch.empty(T, d, dtype=torch.bfloat16 if flags & FT_OUT_BF16 else torch.float32, device=dev)
    if residual_mask is None and want_mask:
        residual_mask = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    _check(lib.ft_moe_combine(_ptr(y_sorted), _ptr(y_shared), _ptr(ids), _ptr(w), _ptr(inv), _ptr(slot_of_expert), T,
                              E, k, d, _ptr(out), _ptr(residual_mask), flags, _stream(stream)))
    return out, (None if residual_mask is None else residual_mask[:T])


# ------------------------------------------------------------------------------------- one layer

class MoELayer:
    """One MoE layer over a device bank with every buffer preallocated for a fixed (T, k).

    forward() enqueues the layer on the current stream and allocates nothing, so it can be replayed
    in a loop or captured into a CUDA/HIP graph by the caller.  mode "layer" makes one ft_moe_layer
    call (the fused decode kernels where they apply); mode "calls" makes the four separate calls."""

    def __init__(self, bank: DeviceBank, slot_of_expert: torch.Tensor, k: int, T: int, shared_slot: int = -1,
                 flags: int = FT_PATH_AUTO, out_bf16: bool = False, mode: str = "layer"):
        if mode not in ("layer", "calls"):
            raise ValueError(f"mode must be 'layer' or 'calls', not {mode!r}")
        if flags & FT_OUT_BF16:  # the output dtype is the layer's own buffer: take the bit from either place
            out_bf16, flags = True, flags & ~FT_OUT_BF16
        dev = bank.w13.device
        E = slot_of_expert.shape[0]
        self.bank, self.slot_of, self.k, self.T, self.E, self.mode = bank, slot_of_expert, k, T, E, mode
        self.shared_slot, self.flags, self.out_flags = shared_slot, flags, FT_OUT_BF16 if out_bf16 else 0
        d = bank.d
        n = max(T * k, 1)
        self.ids = torch.empty(max(T, 1), k, dtype=torch.int32, device=dev)
        self.w = torch.empty(max(T, 1), k, dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.gather = torch.empty(n, dtype=torch.int32, device=dev)
        self.inv = torch.empty(n, dtype=torch.int32, device=dev)
        self.y_sorted = torch.empty(n, d, dtype=torch.bfloat16, device=dev)
        self.y_shared = torch.empty(max(T, 1), d, dtype=torch.bfloat16, device=dev) if shared_slot >= 0 else None
        self.out = torch.empty(max(T, 1), d, dtype=torch.bfloat16 if out_bf16 else torch.float32, device=dev)
        self.mask = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
        if mode == "layer":
            lws = lib.ft_moe_layer_workspace(bank.ref, T, E, k, shared_slot, flags | self.out_flags)
            if lws == 0:
                raise FtError(FT_E_INVAL, f"invalid layer shape T={T} E={E} k={k}")
            self.ws = torch.zeros(lws, dtype=torch.uint8, device=dev)
        else:
            pws = lib.ft_moe_permute_workspace(T, E, k)
            self.perm_ws = torch.empty(max(pws, 256), dtype=torch.uint8, device=dev)
            fws = lib.ft_moe_grouped_ffn_workspace(bank.ref, T, E, k, shared_slot, flags)
            self.ffn_ws = torch.empty(max(fws, 256), dtype=torch.uint8, device=dev)

    def forward_noalloc(self, logits: torch.Tensor, x: torch.Tensor, status: torch.Tensor | None = None, stream=None):
        """The same layer through ft_moe_layer_noalloc: the library's static scratch instead of this
        layer's workspace (status: optional int32 device tensor of one element)."""
        s = _stream(stream)
        _check(lib.ft_moe_layer_noalloc(self.bank.ref, _ptr(self.slot_of), self.shared_slot, _ptr(logits), _ptr(x),
                                        self.T, self.E, self.k, _ptr(self.ids), _ptr(self.w), _ptr(self.counts),
                                        _ptr(self.offsets), _ptr(self.gather), _ptr(self.inv), _ptr(self.y_sorted),
                                        _ptr(self.y_shared), _ptr(self.out), _ptr(self.mask), _ptr(status),
                                        self.flags | self.out_flags, s))
        return self.out[: self.T], self.mask[: self.T]

    def forward_proj(self, x: torch.Tensor, w_router: torch.Tensor, stream=None):
        """The layer from the activations (ft_moe_layer_proj): the router logits x . w_router^T (bf16
        [E][d] router rows) are computed into self.logits, then the layer runs on them.  Mode "layer"."""
        if self.mode != "layer":
            raise ValueError("forward_proj needs mode 'layer'")
        T, E, k = self.T, self.E, self.k
        if getattr(self, "logits", None) is None:
            self.logits = torch.empty(max(T, 1), E, dtype=torch.float32, device=self.out.device)
        _check(lib.ft_moe_layer_proj(self.bank.ref, _ptr(self.slot_of), self.shared_slot, _ptr(x), _ptr(w_router), T,
                                     E, k, _ptr(self.logits), _ptr(self.ids), _ptr(self.w), _ptr(self.counts),
                                     _ptr(self.offsets), _ptr(self.gather), _ptr(self.inv), _ptr(self.y_sorted),
                                     _ptr(self.y_shared), _ptr(self.out), _ptr(self.mask), _ptr(self.ws),
                                     self.ws.numel(), self.flags | self.out_flags, _stream(stream)))
        return self.out[:T], self.mask[:T]

    def status_word(self) -> int:
        """The layer workspace's status word (non-zero: a wait of the fused kernel gave up; the
        unfused path never writes it).  Synchronises."""
        return int(self.ws[:4].view(torch.int32).item()) if self.mode == "layer" else 0

    def forward(self, logits: torch.Tensor, x: torch.Tensor, stream=None):
        T, E, k = self.T, self.E, self.k
        s = _stream(stream)
        if self.mode == "layer":
            _check(lib.ft_moe_layer(self.bank.ref, _ptr(self.slot_of), self.shared_slot, _ptr(logits), _ptr(x), T, E,
                                    k, _ptr(self.ids), _ptr(self.w), _ptr(self.counts), _ptr(self.offsets),
                                    _ptr(self.gather), _ptr(self.inv), _ptr(self.y_sorted), _ptr(self.y_shared),
                                    _ptr(self.out), _ptr(self.mask), _ptr(self.ws), self.ws.numel(),
                                    self.flags | self.out_flags, s))
            return self.out[:T], self.mask[:T]
        _check(lib.ft_moe_route(_ptr(logits), T, E, k, _ptr(self.ids), _ptr(self.w), s))
        _check(lib.ft_moe_permute(_ptr(self.ids), T, E, k, _ptr(self.counts), _ptr(self.offsets), _ptr(self.gather),
                                  _ptr(self.inv), _ptr(self.perm_ws), self.perm_ws.numel(), s))
        _check(lib.ft_moe_grouped_ffn(self.bank.ref, _ptr(self.slot_of), self.shared_slot, _ptr(x), T, E, k,
                                      _ptr(self.offsets), _ptr(self.gather), _ptr(self.y_sorted), _ptr(self.y_shared),
                                      _ptr(self.ffn_ws), self.ffn_ws.numel(), self.flags, s))
        _check(lib.ft_moe_combine(_ptr(self.y_sorted), _ptr(self.y_shared), _ptr(self.ids), _ptr(self.w),
                                  _ptr(self.inv), _ptr(self.slot_of), T, E, k, self.bank.d, _ptr(self.out),
                                  _ptr(self.mask), self.out_flags, s))
        return self.out[:T], self.mask[:T]
