"""Scalar CPU oracle of one Mixture-of-Experts layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The product path (the HIP library and its Python binding) never loads it.

The arithmetic lives in ftoracle.c (plain scalar C, fp32, sums in the order written, built with
-ffp-contract=off and without vectorisation).  This file only loads that library, marshals numpy
arrays, and composes the five steps of the layer in the order the walk-through of the FreeToken
engine gives the request path ("深入FreeToken架构…全链路剖析", section 一: expert dispatch, then the
kernels; section 五: per-format expert banks, hot experts on the GPU, cold experts elsewhere).
`cache_update` is one step of the global LRU expert cache that decides which experts are on the
GPU (ora_cache_update; integer bookkeeping, no arithmetic on values).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ftoracle.c")
_LIB = os.path.join(_HERE, "libftoracle.so")

CFLAGS = ["-O2", "-fno-tree-vectorize", "-fno-tree-slp-vectorize", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-fPIC", "-shared", "-Wall", "-Werror"]

FMT_BF16, FMT_Q4_0, FMT_MXFP4, FMT_FP8_B128, FMT_NVFP4 = 0, 1, 2, 3, 4


def build(extra_flags=(), out=_LIB) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *extra_flags, _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def _load(path=None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    i = ctypes.c_int
    lib.ora_dequant.argtypes = [i, P, P, i, i, i, i, P]
    lib.ora_route.argtypes = [P, i, i, i, P, P]
    lib.ora_router_logits.argtypes = [P, P, i, i, i, P]
    lib.ora_permute.argtypes = [P, i, i, i, P, P, P, P]
    lib.ora_swiglu_ffn.argtypes = [P, i, i, i, P, P, P, P]
    lib.ora_combine.argtypes = [P, P, P, P, P, P, i, i, i, i, P, i, P, P]
    lib.ora_cache_update.argtypes = [P, i, i, i, ctypes.c_float, P, P, P, P, P, P, P]
    for f in ("ora_bf16_value", "ora_fp16_value"):
        getattr(lib, f).argtypes = [ctypes.c_uint16]
        getattr(lib, f).restype = ctypes.c_float
    for f in ("ora_e2m1_value", "ora_e4m3_value", "ora_e8m0_value"):
        getattr(lib, f).argtypes = [ctypes.c_uint]
        getattr(lib, f).restype = ctypes.c_float
    return lib


def _p(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _np(t, dtype=None):
    """torch tensor or array -> C-contiguous numpy array on the host."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if str(t.dtype) == "torch.bfloat16":
            import torch
            t = t.view(torch.int16)
        t = t.numpy()
    a = np.ascontiguousarray(t)
    if dtype is not None:
        a = a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments")


# ------------------------------------------------------------------------- element decoders

def e2m1_value(code: int, lib=None) -> float:
    return (lib or _load()).ora_e2m1_value(code)


def e4m3_value(code: int, lib=None) -> float:
    return (lib or _load()).ora_e4m3_value(code)


def e8m0_value(code: int, lib=None) -> float:
    return (lib or _load()).ora_e8m0_value(code)


def fp16_value(bits: int, lib=None) -> float:
    return (lib or _load()).ora_fp16_value(bits)


def bf16_value(bits: int, lib=None) -> float:
    return (lib or _load()).ora_bf16_value(bits)


# ------------------------------------------------------------------------- steps

def dequant(fmt: int, codes, scales, rows: int, K: int, row0: int = 0, nrows: int | None = None,
            lib=None) -> np.ndarray:
    """fp32 [nrows][K] decode of rows [row0, row0+nrows) of one stored matrix."""
    nrows = rows - row0 if nrows is None else nrows
    c = _np(codes)
    s = _np(scales)
    out = np.empty((nrows, K), np.float32)
    _check((lib or _load()).ora_dequant(fmt, _p(c), _p(s), rows, K, row0, nrows, _p(out)), "dequant")
    return out


def route(logits, k: int, lib=None):
    """ids int32 [T][k], w fp32 [T][k]."""
    L = _np(logits, np.float32)
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check((lib or _load()).ora_route(_p(L), T, E, k, _p(ids), _p(w)), "route")
    return ids, w


def router_logits(x_bf16, w_router_bf16, lib=None):
    """fp64 [T][E] router logits x . w_router^T of bf16 activations [T][d] and router rows [E][d]
    (torch bf16 tensors or uint16 bit arrays)."""
    x = _bf16_bits(x_bf16)
    wr = _bf16_bits(w_router_bf16)
    T, d = x.shape
    E = wr.shape[0]
    assert wr.shape[1] == d
    out = np.empty((T, E), np.float64)
    _check((lib or _load()).ora_router_logits(_p(x), _p(wr), T, d, E, _p(out)), "router_logits")
    return out


def _bf16_bits(a) -> np.ndarray:
    """uint16 bit array of a torch bf16 tensor or of an integer array of bf16 bits."""
    if hasattr(a, "view") and hasattr(a, "dtype") and "bfloat16" in str(getattr(a, "dtype", "")):
        import torch  # noqa: F401  (only when given a torch tensor)
        return np.ascontiguousarray(a.detach().cpu().view(torch.int16).numpy().view(np.uint16))
    return np.ascontiguousarray(np.asarray(a).astype(np.uint16))


def permute(ids, E: int, lib=None):
    """counts [E], offsets [E+1], gather [T*k], inv [T*k] (all int32)."""
    a = _np(ids, np.int32)
    T, k = a.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    gather = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    _check((lib or _load()).ora_permute(_p(a), T, E, k, _p(counts), _p(offsets), _p(gather), _p(inv)),
           "permute")
    return counts, offsets, gather, inv


class CacheState:
    """Host copy of the expert cache's tables: slot_of_expert [E], expert_of_slot [S] (int32, -1 =
    none), last_use [S] and tick (uint32).  A fresh state has every slot empty."""

    def __init__(self, E: int, S: int):
        self.slot_of_expert = np.full(E, -1, np.int32)
        self.expert_of_slot = np.full(S, -1, np.int32)
        self.last_use = np.zeros(S, np.uint32)
        self.tick = np.zeros(1, np.uint32)

    def copy(self):
        c = CacheState.__new__(CacheState)
        for f in ("slot_of_expert", "expert_of_slot", "last_use", "tick"):
            setattr(c, f, getattr(self, f).copy())
        return c


def cache_update(counts, state: CacheState, max_loads: int, load_fraction: float = 0.0, lib=None,
                 with_load_slot: bool = False):
    """One step of the global LRU expert cache on `state` (updated in place).

    Returns (compute_slot int32 [E], loads int32 [n][2] of (expert, slot)), and load_slot int32 [E]
    after them when with_load_slot."""
    c = _np(counts, np.int32)
    E, S = c.shape[0], state.expert_of_slot.shape[0]
    compute_slot = np.empty(E, np.int32)
    load_slot = np.empty(E, np.int32)
    loads = np.empty(2 * max(max_loads, 1), np.int32)
    n = (lib or _load()).ora_cache_update(_p(c), E, S, max_loads, float(load_fraction), _p(state.slot_of_expert),
                                          _p(state.expert_of_slot), _p(state.last_use), _p(state.tick),
                                          _p(compute_slot), _p(load_slot), _p(loads))
    if n < 0:
        raise ValueError("oracle cache_update rejected its arguments")
    out = (compute_slot, loads[:2 * n].reshape(n, 2).copy())
    return out + (load_slot,) if with_load_slot else out


def swiglu_ffn(x_f32, w13_f32, w2_f32, lib=None):
    """h fp32 [n][I], y fp32 [n][d] for input rows x_f32 [n][d]."""
    x = _np(x_f32, np.float32)
    w13 = _np(w13_f32, np.float32)
    w2 = _np(w2_f32, np.float32)
    n, d = x.shape
    I = w13.shape[0] // 2
    h = np.empty((n, I), np.float32)
    y = np.empty((n, d), np.float32)
    _check((lib or _load()).ora_swiglu_ffn(_p(x), n, d, I, _p(w13), _p(w2), _p(h), _p(y)), "ffn")
    return h, y


def combine(y_sorted, y_shared, ids, w, inv, slot_of, d: int, tokens=None, lib=None):
    """out fp32 [T][d] (rows of tokens not listed stay zero) and mask uint32 [T]."""
    ids = _np(ids, np.int32)
    T, k = ids.shape
    E = len(slot_of)
    ys = _np(y_sorted, np.float32)
    ysh = _np(y_shared, np.float32)
    wv = _np(w, np.float32)
    iv = _np(inv, np.int32)
    so = _np(slot_of, np.int32)
    tk = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, np.int32))
    out = np.zeros((T, d), np.float32)
    mask = np.zeros(T, np.uint32)
    _check((lib or _load()).ora_combine(_p(ys), _p(ysh), _p(ids), _p(wv), _p(iv), _p(so), T, E, k, d,
                                        _p(tk), 0 if tk is None else len(tk), _p(out), _p(mask)),
           "combine")
    return out, mask


def bf16_to_f32(x) -> np.ndarray:
    """Exact widening of bf16 activations (given as a torch bf16 tensor or uint16/int16 bits)."""
    a = _np(x)
    return (a.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)


def dequant_slot(bank, slot: int, lib=None):
    """fp32 W13 [2I][d] and W2 [d][I] of one slot of a canonical bank (synth.Bank or alike)."""
    d, I, fmt = bank.d, bank.I, bank.fmt
    s13 = None if bank.s13 is None else bank.s13[slot]
    s2 = None if bank.s2 is None else bank.s2[slot]
    w13 = dequant(fmt, bank.w13[slot], s13, 2 * I, d, lib=lib)
    w2 = dequant(fmt, bank.w2[slot], s2, d, I, lib=lib)
    return w13, w2


# ------------------------------------------------------------------------- the layer

CHUNK_ROWS = 256   # rows per job of the threaded layer


def layer(logits, x_bf16, bank, slot_of, k: int, shared_slot: int = -1, tokens=None, lib=None, workers: int = 1):
    """One MoE layer, optionally only for a sample of tokens.

    Returns a dict with ids, w, counts, offsets, gather, inv (whole layer), and for the computed
    tokens: mask [T], out [T][d] (zero rows for tokens not computed), y_pos (sorted positions
    computed), y_rows fp32 [len(y_pos)][d], y_shared fp32 [T][d] or None.
    `workers` > 1 runs the expert groups on that many threads (the C calls release the GIL), large
    groups cut into runs of at most CHUNK_ROWS rows so that a skewed routing still spreads over the
    threads; every row's arithmetic is the same as with one worker (rows are independent).
    """
    lib = lib or _load()
    L = _np(logits, np.float32)
    T, E = L.shape
    d = bank.d
    so = _np(slot_of, np.int32)
    ids, w = route(L, k, lib=lib)
    counts, offsets, gather, inv = permute(ids, E, lib=lib)
    want = np.ones(T, bool) if tokens is None else np.isin(np.arange(T), np.asarray(tokens))
    xf = bf16_to_f32(x_bf16)
    jobs = []
    for e in range(E):
        s = int(so[e])
        if s < 0 or counts[e] == 0:
            continue
        pos = np.arange(offsets[e], offsets[e + 1])
        pos = pos[want[gather[pos] // k]]
        step = CHUNK_ROWS if workers > 1 else max(len(pos), 1)
        for r0 in range(0, len(pos), step):
            jobs.append((s, pos[r0:r0 + step]))

    def run(job):
        s, pos = job
        w13, w2 = dequant_slot(bank, s, lib=lib)
        return swiglu_ffn(xf[gather[pos] // k], w13, w2, lib=lib)[1]

    if workers > 1 and len(jobs) > 1:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            ys = list(ex.map(run, jobs))
    else:
        ys = [run(j) for j in jobs]
    y_pos_all = [pos for _, pos in jobs]
    y_rows_all = ys
    y_pos = np.concatenate(y_pos_all) if y_pos_all else np.zeros(0, np.int64)
    y_rows = np.concatenate(y_rows_all) if y_rows_all else np.zeros((0, d), np.float32)
    y_shared = None
    if shared_slot >= 0:
        y_shared = np.zeros((T, d), np.float32)
        w13, w2 = dequant_slot(bank, shared_slot, lib=lib)
        tok = np.nonzero(want)[0]
        _, ysh = swiglu_ffn(xf[tok], w13, w2, lib=lib)
        y_shared[tok] = ysh
    # compact y_sorted: local row index of each computed sorted position
    local = np.zeros(T * k, np.int32)
    local_inv = np.zeros(T * k, np.int32)
    local[y_pos] = np.arange(len(y_pos), dtype=np.int32)
    computed = np.zeros(T * k, bool)
    computed[y_pos] = True
    flat_ok = computed[inv]
    local_inv[flat_ok] = local[inv[flat_ok]]
    tok_list = np.nonzero(want)[0].astype(np.int32)
    out, mask = combine(y_rows if len(y_rows) else np.zeros((1, d), np.float32), y_shared, ids, w,
                        local_inv, so, d, tokens=tok_list, lib=lib)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, gather=gather, inv=inv, mask=mask,
                out=out, y_pos=y_pos, y_rows=y_rows, y_shared=y_shared, tokens=tok_list)
