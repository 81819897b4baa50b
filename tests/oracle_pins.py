"""Pins of the CPU oracle to things other than itself.

Each pin takes a loaded oracle library (`oracle._load()` or a deliberately broken build of it)
and raises AssertionError when the oracle disagrees with brute force, a library routine, a
published format table, a closed form or an invariant.  tests/test_oracle_pins.py runs them on
the real oracle; tests/test_oracle_mutants.py checks that every planted mistake trips at least
one of them.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _tie_logits(rng, T, E):
    """Logits from a small integer set so that ties are common, plus a few -inf."""
    L = rng.integers(-3, 4, size=(T, E)).astype(np.float32) * 0.5
    L[rng.random((T, E)) < 0.05] = -np.inf
    L[:, 0] = np.where(rng.random(T) < 0.3, -0.0, L[:, 0])
    return L


def _precedes(a, b, row):
    """Route order: larger logit first, equal logits by lower expert index (IEEE ==, so -0 == +0)."""
    return row[a] > row[b] or (row[a] == row[b] and a < b)


# ------------------------------------------------------------------------------ route

def pin_route_bruteforce(lib):
    """ids = the unique k-subset whose members all precede every non-member, ordered by precedence."""
    rng = np.random.default_rng(11)
    for E in range(1, 11):
        for k in range(1, min(4, E) + 1):
            L = _tie_logits(rng, 24, E)
            ids, _ = oracle.route(L, k, lib=lib)
            for t in range(L.shape[0]):
                row = L[t]
                winners = [S for S in itertools.combinations(range(E), k)
                           if all(_precedes(a, b, row) for a in S for b in range(E) if b not in S)]
                assert len(winners) == 1, (E, k, t)
                S = list(winners[0])
                ordered = sorted(S, key=lambda e: (-float(row[e]), e))
                assert list(ids[t]) == ordered, (E, k, t, row, ids[t], ordered)


def pin_route_special_cases(lib):
    rng = np.random.default_rng(12)
    # all-equal logits -> ids 0..k-1
    ids, w = oracle.route(np.full((5, 9), 0.25, np.float32), 4, lib=lib)
    assert (ids == np.arange(4)).all()
    assert (w == np.float32(0.25)).all()          # 1/k exactly for a power-of-two k
    # k = E -> the whole descending order (numpy lexsort as the library cross-check)
    L = _tie_logits(rng, 16, 7)
    L[np.isinf(L)] = -5.0
    ids, _ = oracle.route(L, 7, lib=lib)
    for t in range(16):
        assert list(ids[t]) == list(np.lexsort((np.arange(7), -L[t].astype(np.float64))))
    # adding a constant to a row leaves the ids unchanged
    L = rng.standard_normal((32, 12)).astype(np.float32)
    a, _ = oracle.route(L, 3, lib=lib)
    b, _ = oracle.route(L + np.float32(3.0), 3, lib=lib)
    assert (a == b).all()
    # k = 1 -> weight exactly 1
    _, w = oracle.route(L, 1, lib=lib)
    assert (w == 1.0).all()


def pin_route_weights_float64(lib):
    """Weights = float64 softmax, restricted to the chosen ids and renormalised, within 1e-6."""
    rng = np.random.default_rng(13)
    for E, k, scale in ((8, 2, 1.0), (64, 8, 1.0), (256, 8, 3.0), (5, 5, 1.0)):
        L = (rng.standard_normal((40, E)) * scale).astype(np.float32)
        ids, w = oracle.route(L, k, lib=lib)
        L64 = L.astype(np.float64)
        p = np.exp(L64 - L64.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
        ref = sel / sel.sum(axis=1, keepdims=True)
        assert np.abs(w - ref).max() <= 1e-6, np.abs(w - ref).max()
        assert np.abs(w.astype(np.float64).sum(axis=1) - 1.0).max() <= 1e-6
        assert (np.diff(w, axis=1) <= 0).all()   # descending logits give non-increasing weights


# ------------------------------------------------------------------------------ permute

def pin_permute(lib):
    rng = np.random.default_rng(14)
    for T, E, k in ((1, 4, 1), (17, 8, 2), (64, 10, 4), (300, 128, 8), (0, 5, 2)):
        ids = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
        if T > 5:   # skew: many tokens on expert 0
            ids[: T // 2, 0] = 0
            ids[: T // 2, 1:] = np.stack([rng.permutation(np.arange(1, E))[: k - 1] for _ in range(T // 2)])
        counts, offsets, gather, inv = oracle.permute(ids, E, lib=lib)
        flat = ids.reshape(-1)
        assert (counts == np.bincount(flat, minlength=E)).all()
        assert counts.sum() == T * k and offsets[0] == 0 and offsets[E] == T * k
        assert (np.diff(offsets) == counts).all()
        ref = np.argsort(flat, kind="stable")       # library cross-check: stable sort by expert
        assert (gather == ref).all()
        assert (np.sort(gather) == np.arange(T * k)).all()   # bijection
        assert (inv[gather] == np.arange(T * k)).all()
        for e in range(E):
            g = gather[offsets[e]:offsets[e + 1]]
            assert (flat[g] == e).all() and (np.diff(g) > 0).all()


# ------------------------------------------------------------------------------ element decoders

def pin_decoder_tables(lib):
    for code, val in _golden("e2m1_values.txt"):
        got = oracle.e2m1_value(int(code), lib=lib)
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got)
    for code, val in _golden("e4m3_special.txt"):
        got = oracle.e4m3_value(int(code, 16), lib=lib)
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got)
    # all 256 e4m3 codes against torch's float8_e4m3fn decode (library routine)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_value(c, lib=lib) for c in range(256)], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)) or \
        np.array_equal(np.nan_to_num(got, nan=7.0), np.nan_to_num(ref, nan=7.0))
    # all 65536 fp16 codes against numpy's float16 (library routine), bit for bit (NaN payload aside)
    bits = np.arange(65536, dtype=np.uint32)
    ref16 = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    got16 = np.array([oracle.fp16_value(int(b), lib=lib) for b in bits], np.float32)
    nan = np.isnan(ref16)
    assert (np.isnan(got16) == nan).all()
    assert np.array_equal(got16[~nan].view(np.uint32), ref16[~nan].view(np.uint32))
    # E8M0 = 2^(s-127), 0xFF = NaN; bf16 = upper half of fp32
    for s in range(255):
        assert oracle.e8m0_value(s, lib=lib) == 2.0 ** (s - 127), s
    assert math.isnan(oracle.e8m0_value(255, lib=lib))
    for b in (0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x8000):
        ref = np.array([b << 16], np.uint32).view(np.float32)[0]
        assert oracle.bf16_value(b, lib=lib) == ref


def _exact_q4_0_weights(rng, rows, K):
    """Weights exactly representable in Q4_0: per block scale s = m * 2^-22 (m odd in [1024, 2048), so s
    is an exact normal fp16) and integers q-8 in [-8, 7] with the block's extreme value -8 present (so the encoder
    recovers s exactly)."""
    nb = K // 32
    s = (rng.integers(1024, 2048, size=(rows, nb)) | 1).astype(np.float64) * 2.0 ** -22
    q = rng.integers(-7, 8, size=(rows, nb, 32)).astype(np.float64)
    q[..., rng.integers(0, 32)] = -8.0
    return (q * s[..., None]).reshape(rows, K)


def pin_dequant_roundtrip(lib):
    """Encoding exactly representable weights with the input encoders and decoding them with the
    oracle gives the weights back bit for bit, for every format."""
    rng = np.random.default_rng(15)
    rows, K = 256, 256
    # bf16: any bf16 value
    w = torch.from_numpy(rng.standard_normal((rows, K)).astype(np.float32)).to(torch.bfloat16).float()
    c, _ = synth.encode_bf16(w)
    assert np.array_equal(oracle.dequant(0, c, None, rows, K, lib=lib), w.numpy())
    # Q4_0
    w = _exact_q4_0_weights(rng, rows, K).astype(np.float32)
    c, _ = synth.encode_q4_0(torch.from_numpy(w))
    assert np.array_equal(oracle.dequant(1, c, None, rows, K, lib=lib), w)
    # MXFP4: e2m1 grid values times 2^k, block max magnitude 4 or 6 so the shared exponent is k
    grid = np.array([float(v) for _, v in _golden("e2m1_values.txt")], np.float64)
    v = grid[rng.integers(0, 16, size=(rows, K // 32, 32))]
    v[..., 3] = rng.choice([4.0, 6.0, -4.0, -6.0], size=(rows, K // 32))
    e = rng.integers(-12, 3, size=(rows, K // 32, 1)).astype(np.float64)
    w = (v * 2.0 ** e).reshape(rows, K).astype(np.float32)
    c, s = synth.encode_mxfp4(torch.from_numpy(w))
    got = oracle.dequant(2, c, s, rows, K, lib=lib)
    assert np.array_equal(got, w), np.abs(got - w).max()
    # FP8-B128: e4m3 values times a power-of-two block scale, with +-448 in every block
    codes = rng.integers(0, 256, size=(rows, K)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    vals = vals.reshape(rows // 128, 128, K // 128, 128)
    vals[:, 5, :, 7] = 448.0
    sc = 2.0 ** rng.integers(-10, -4, size=(rows // 128, 1, K // 128, 1)).astype(np.float64)
    w = (vals * sc).reshape(rows, K).astype(np.float32)
    c, s = synth.encode_fp8_b128(torch.from_numpy(w))
    got = oracle.dequant(3, c, s, rows, K, lib=lib)
    assert np.array_equal(got, w), np.abs(got - w).max()
    # NVFP4: e2m1 grid values times an e4m3 block scale times a tensor scale t.  With +-6 in every
    # 16-block and amax = 6 * 448 * t in the matrix, the encoder recovers t and every block scale
    # (t a power of two so that amax / (448 * 6) is t exactly; block scales e4m3 values in [1, 448])
    t = 2.0 ** -9
    v = grid[rng.integers(0, 16, size=(rows, K // 16, 16))]
    v[..., 5] = rng.choice([6.0, -6.0], size=(rows, K // 16))
    sc_codes = rng.integers(0x38, 0x7F, size=(rows, K // 16, 1)).astype(np.uint8)  # e4m3 1.0 .. 448
    sc_codes[0, 0, 0] = 0x7E                                                       # 448 somewhere
    bs = torch.from_numpy(sc_codes).view(torch.float8_e4m3fn).double().numpy()
    w = (v * bs * t).reshape(rows, K).astype(np.float32)
    c, s = synth.encode_nvfp4(torch.from_numpy(w))
    got = oracle.dequant(4, c, s, rows, K, lib=lib)
    assert np.array_equal(got, w), np.abs(got - w).max()


def pin_dequant_layouts(lib):
    """Hand-built blocks with known element positions (GGUF Q4_0 nibble order, OCP MX packing,
    128x128 FP8 block grid) decode to the values the format definitions give them."""
    # Q4_0: one row, two blocks; block b has scale 2^-b (fp16), element i gets code (i % 16)
    blk = np.zeros((1, 2, 18), np.uint8)
    ref = np.zeros((1, 64), np.float64)
    for b in range(2):
        blk[0, b, 0:2] = np.array([2.0 ** -b], np.float16).view(np.uint8)
        for i in range(32):
            q = (i * 7 + b) % 16
            byte = 2 + (i % 16)
            blk[0, b, byte] |= (q << 4) if i >= 16 else q
            ref[0, 32 * b + i] = (q - 8) * 2.0 ** -b
    assert np.array_equal(oracle.dequant(1, blk, None, 1, 64, lib=lib), ref.astype(np.float32))
    # MXFP4: element j of the row gets code j % 16; scales 2^(s-127) with s = 125, 130
    codes = np.array([(2 * i % 16) | (((2 * i + 1) % 16) << 4) for i in range(32)], np.uint8)[None]
    sc = np.array([[125, 130]], np.uint8)
    grid = np.array([float(v) for _, v in _golden("e2m1_values.txt")])
    ref = np.array([grid[j % 16] * 2.0 ** (int(sc[0, j // 32]) - 127) for j in range(64)])[None]
    assert np.array_equal(oracle.dequant(2, codes, sc, 1, 64, lib=lib), ref.astype(np.float32))
    # NVFP4: same code layout as MXFP4; 16-element blocks with e4m3 scales 0x30 (0.5), 0x40 (2.0),
    # 0x3C (1.5), 0x44 (3.0); tensor scale 0.25 stored after the block scales
    bsc = np.array([[0x30, 0x40, 0x3C, 0x44]], np.uint8)
    tail = np.array([0.25], np.float32).view(np.uint8)
    ns = np.concatenate([bsc.reshape(-1), tail])
    bval = [0.5, 2.0, 1.5, 3.0]
    ref = np.array([0.25 * grid[j % 16] * bval[j // 16] for j in range(64)])[None]
    assert np.array_equal(oracle.dequant(4, codes, ns, 1, 64, lib=lib), ref.astype(np.float32))
    # FP8-B128: 256x256 of code 0x38 (1.0); block (rb, cb) has scale 1 + rb + 2cb
    codes = np.full((256, 256), 0x38, np.uint8)
    sc = np.array([[1.0, 3.0], [2.0, 4.0]], np.float32)
    got = oracle.dequant(3, codes, sc, 256, 256, lib=lib)
    ref = np.repeat(np.repeat(sc, 128, axis=0), 128, axis=1)
    assert np.array_equal(got, ref)
    # a partial row range decodes the same rows
    assert np.array_equal(oracle.dequant(3, codes, sc, 256, 256, row0=130, nrows=3, lib=lib), ref[130:133])


# ------------------------------------------------------------------------------ FFN and layer

def pin_ffn_float64(lib):
    """SwiGLU against float64 numpy matmuls on the same fp32 inputs: rel-L2 <= 1e-5."""
    rng = np.random.default_rng(16)
    for n, d, I in ((5, 64, 48), (3, 256, 96), (1, 32, 32)):
        x = rng.standard_normal((n, d)).astype(np.float32)
        w13 = (rng.standard_normal((2 * I, d)) * 0.05).astype(np.float32)
        w2 = (rng.standard_normal((d, I)) * 0.05).astype(np.float32)
        h, y = oracle.swiglu_ffn(x, w13, w2, lib=lib)
        x64, w64, d64 = x.astype(np.float64), w13.astype(np.float64), w2.astype(np.float64)
        g = x64 @ w64[:I].T
        u = x64 @ w64[I:].T
        h64 = g / (1.0 + np.exp(-g)) * u
        y64 = h64 @ d64.T
        assert np.linalg.norm(h - h64) <= 1e-5 * np.linalg.norm(h64)
        assert np.linalg.norm(y - y64) <= 1e-5 * np.linalg.norm(y64)
    # x = 0 -> y = 0; W_down = 0 -> y = 0
    _, y = oracle.swiglu_ffn(np.zeros((2, 64), np.float32),
                             (rng.standard_normal((64, 64)) * 0.1).astype(np.float32),
                             (rng.standard_normal((64, 32)) * 0.1).astype(np.float32), lib=lib)
    assert (y == 0).all()
    _, y = oracle.swiglu_ffn(rng.standard_normal((2, 64)).astype(np.float32),
                             (rng.standard_normal((64, 64)) * 0.1).astype(np.float32),
                             np.zeros((64, 32), np.float32), lib=lib)
    assert (y == 0).all()


def _tiny_layer_inputs(rng, T, d, E, k, I, fmt=0, identical=False):
    w = synth.Workload("pin", 99, T=T, d=d, E=E, k=k, I=I, fmt=fmt)
    bank = synth.empty_bank(fmt, E, d, I)
    w13 = torch.from_numpy((rng.standard_normal((2 * I, d)) * 0.05).astype(np.float32))
    w2 = torch.from_numpy((rng.standard_normal((d, I)) * 0.05).astype(np.float32))
    for s in range(E):
        if not identical:
            w13 = torch.from_numpy((rng.standard_normal((2 * I, d)) * 0.05).astype(np.float32))
            w2 = torch.from_numpy((rng.standard_normal((d, I)) * 0.05).astype(np.float32))
        synth.fill_slot(bank, s, w13, w2)
    L = rng.standard_normal((T, E)).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    return w, bank, L, x


def pin_layer_identical_experts(lib):
    """All experts identical -> the layer equals one dense SwiGLU FFN of x (sum of weights is 1)."""
    rng = np.random.default_rng(17)
    for fmt in (0, 1, 2):
        w, bank, L, x = _tiny_layer_inputs(rng, 12, 64, 6, 3, 64, fmt=fmt, identical=True)
        r = oracle.layer(L, x, bank, np.arange(6, dtype=np.int32), 3, lib=lib)
        w13, w2 = oracle.dequant_slot(bank, 0, lib=lib)
        _, dense = oracle.swiglu_ffn(oracle.bf16_to_f32(x), w13, w2, lib=lib)
        tol = 8 * 2.0 ** -24 * np.abs(dense).max()
        assert np.abs(r["out"] - dense).max() <= tol, np.abs(r["out"] - dense).max()


def pin_layer_float64(lib):
    """Whole layer against a float64 numpy evaluation of the same definition (library matmuls,
    numpy stable sort for the grouping) on fp32-decoded weights: rel-L2 <= 1e-5."""
    rng = np.random.default_rng(18)
    T, d, E, k, I = 20, 64, 6, 2, 32
    w, bank, L, x = _tiny_layer_inputs(rng, T, d, E, k, I, fmt=0)
    slot_of = np.array([2, -1, 0, 1, 5, 4], np.int32)     # expert 1 not resident
    r = oracle.layer(L, x, bank, slot_of, k, shared_slot=3, lib=lib)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    W = [[a.astype(np.float64) for a in oracle.dequant_slot(bank, s, lib=lib)] for s in range(E)]

    def ffn(xr, s):
        w13, w2 = W[s]
        g = xr @ w13[:I].T
        return (g / (1 + np.exp(-g)) * (xr @ w13[I:].T)) @ w2.T

    out = ffn(xf, 3)
    for t in range(T):
        order = np.lexsort((np.arange(E), -L[t].astype(np.float64)))[:k]
        p = np.exp(L[t].astype(np.float64) - L[t].max())
        wt = p[order] / p[order].sum()
        for j, e in enumerate(order):
            if slot_of[e] >= 0:
                out[t] += wt[j] * ffn(xf[t:t + 1], slot_of[e])[0]
        assert r["mask"][t] == sum(1 << j for j, e in enumerate(order) if slot_of[e] < 0)
    assert np.linalg.norm(r["out"] - out) <= 1e-5 * np.linalg.norm(out)


def pin_layer_sampled_threaded(lib, ora=oracle):
    """The layer restricted to a token sample and run on several threads (the form the full-size GPU
    tests check against) equals the whole single-threaded layer on the sampled tokens, bit for bit:
    same rows of out, mask and y_shared, zero rows elsewhere, and y rows for exactly the resident
    pairs of the sampled tokens (their sorted positions from the definition of the permutation).
    `ora` is the oracle module (a planted copy in the mutant tests)."""
    rng = np.random.default_rng(20)
    old_rows = ora.CHUNK_ROWS
    ora.CHUNK_ROWS = 5            # groups of these tiny layers span several threaded runs
    try:
        for fmt, (T, d, E, k, I) in ((0, (40, 64, 7, 3, 32)), (1, (33, 64, 9, 2, 64)), (2, (24, 32, 5, 4, 32))):
            w, bank, L, x = _tiny_layer_inputs(rng, T, d, E + 1, k, I, fmt=fmt)    # slot E: shared expert
            L = L[:, :E].copy()
            slot_of = rng.permutation(E).astype(np.int32)
            slot_of[rng.choice(E, size=2, replace=False)] = -1                     # two experts not resident
            full = ora.layer(L, x, bank, slot_of, k, shared_slot=E, lib=lib)
            ids_flat = full["ids"].reshape(-1)
            for S in (rng.choice(T, size=T // 3, replace=False), np.array([0]), np.array([T - 1]), np.arange(T)):
                S = np.sort(S)
                part = ora.layer(L, x, bank, slot_of, k, shared_slot=E, tokens=S, lib=lib, workers=4)
                for key in ("ids", "w", "counts", "offsets", "gather", "inv"):
                    assert np.array_equal(part[key], full[key]), key
                assert np.array_equal(part["tokens"], S)
                inS = np.zeros(T, bool)
                inS[S] = True
                assert np.array_equal(part["out"][inS], full["out"][inS])
                assert (part["out"][~inS] == 0).all()
                assert np.array_equal(part["mask"][inS], full["mask"][inS]) and (part["mask"][~inS] == 0).all()
                assert np.array_equal(part["y_shared"][inS], full["y_shared"][inS])
                assert (part["y_shared"][~inS] == 0).all()
                want = [p for p in range(T * k) if inS[full["gather"][p] // k] and slot_of[ids_flat[full["gather"][p]]] >= 0]
                assert part["y_pos"].tolist() == want
                where = {int(p): i for i, p in enumerate(full["y_pos"])}
                rows = [where[int(p)] for p in part["y_pos"]]
                assert np.array_equal(part["y_rows"], full["y_rows"][rows])
    finally:
        ora.CHUNK_ROWS = old_rows


def pin_combine_cases(lib):
    rng = np.random.default_rng(19)
    T, d, E, k = 9, 32, 5, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    _, _, _, inv = oracle.permute(ids, E, lib=lib)
    y = rng.standard_normal((T * k, d)).astype(np.float32)
    ysh = rng.standard_normal((T, d)).astype(np.float32)
    # nothing resident: out = y_shared, mask = all k bits
    out, mask = oracle.combine(y, ysh, ids, w, inv, np.full(E, -1, np.int32), d, lib=lib)
    assert np.array_equal(out, ysh) and (mask == (1 << k) - 1).all()
    out, mask = oracle.combine(y, None, ids, w, inv, np.full(E, -1, np.int32), d, lib=lib)
    assert (out == 0).all()
    # everything resident: mask 0; one-hot k=1 with weight 1 returns y itself
    _, mask = oracle.combine(y, None, ids, w, inv, np.arange(E, dtype=np.int32), d, lib=lib)
    assert (mask == 0).all()
    ids1 = ids[:, :1].copy()
    _, _, _, inv1 = oracle.permute(ids1, E, lib=lib)
    out, _ = oracle.combine(y[:T], None, ids1, np.ones((T, 1), np.float32), inv1,
                            np.arange(E, dtype=np.int32), d, lib=lib)
    assert np.array_equal(out, y[:T][inv1])
    # weighted sum in float64 (two experts resident, one not)
    slot_of = np.array([0, 1, -1, 3, 4], np.int32)
    out, mask = oracle.combine(y, None, ids, w, inv, slot_of, d, lib=lib)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if slot_of[ids[t, j]] >= 0:
                ref[t] += float(w[t, j]) * y[inv[t * k + j]].astype(np.float64)
        assert mask[t] == sum(1 << j for j in range(k) if slot_of[ids[t, j]] < 0)
    assert np.abs(out - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())


def _bf16_bits_of(vals):
    """bf16 bit patterns of values that bf16 holds exactly."""
    f = np.asarray(vals, np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def pin_router_logits_worked_example(lib):
    """A hand-computed example: two tokens, three columns, two experts."""
    x = _bf16_bits_of([[1.0, 2.0, -3.0], [0.5, -0.25, 4.0]])
    wr = _bf16_bits_of([[1.0, 1.0, 1.0], [0.5, 0.0, 0.25]])
    got = oracle.router_logits(x, wr, lib=lib)
    # token 0: 1 + 2 - 3 = 0 and 0.5 + 0 - 0.75 = -0.25; token 1: 0.5 - 0.25 + 4 = 4.25 and
    # 0.25 + 0 + 1 = 1.25
    assert np.array_equal(got, np.array([[0.0, -0.25], [4.25, 1.25]]))


def pin_router_logits_one_hot(lib):
    """A router row with a single 1 at column c picks x[:, c] exactly; a transposed or shifted
    operand would not."""
    rng = np.random.default_rng(11)
    T, d, E = 5, 64, 7
    xf = rng.standard_normal((T, d)).astype(np.float32)
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)
    cols = rng.permutation(d)[:E]
    w = np.zeros((E, d), np.float32)
    w[np.arange(E), cols] = 1.0
    got = oracle.router_logits(x, _bf16_bits_of(w), lib=lib)
    xw = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, xw[:, cols])


def pin_router_logits_exact_sum(lib):
    """Against the exact rational sum (brute force with fractions): within the rounding bound of a
    double-precision sum of d terms."""
    from fractions import Fraction
    rng = np.random.default_rng(12)
    T, d, E = 3, 48, 4
    x = (rng.standard_normal((T, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wr = ((0.02 * rng.standard_normal((E, d))).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = oracle.router_logits(x, wr, lib=lib)
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    wv = (wr.astype(np.uint32) << 16).view(np.float32)
    for t in range(T):
        for e in range(E):
            terms = [Fraction(float(xv[t, c])) * Fraction(float(wv[e, c])) for c in range(d)]
            exact = sum(terms, Fraction(0))
            bound = d * 2.0 ** -53 * float(sum(abs(v) for v in terms))
            assert abs(Fraction(got[t, e]) - exact) <= Fraction(bound)


# ------------------------------------------------------------------------------ expert cache

def pin_cache_textbook_lru(lib):
    """One demanded expert and at most one load per step: the cache is then a textbook LRU cache
    of S entries (on a miss with every entry taken, the least recently requested one goes), so
    the resident set, the hits and the misses must agree with an OrderedDict LRU step by step."""
    from collections import OrderedDict
    rng = np.random.default_rng(31)
    for E, S, steps in ((12, 4, 300), (7, 1, 60), (5, 5, 50), (40, 9, 500)):
        st = oracle.CacheState(E, S)
        ref = OrderedDict()
        ranks = np.minimum(rng.geometric(0.25, size=steps) - 1, E - 1)   # skewed: hits and misses
        reqs = rng.permutation(E)[ranks]
        for step, e in enumerate(reqs):
            e = int(e)
            counts = np.zeros(E, np.int32)
            counts[e] = 1 + step % 3
            hit = e in ref
            if hit:
                ref.move_to_end(e)
            else:
                if len(ref) == S:
                    ref.popitem(last=False)
                ref[e] = True
            cs, loads = oracle.cache_update(counts, st, 1, lib=lib)
            assert set(np.flatnonzero(st.slot_of_expert >= 0).tolist()) == set(ref), (E, S, step)
            if hit:
                assert len(loads) == 0 and cs[e] == st.slot_of_expert[e] >= 0
            else:
                assert len(loads) == 1 and loads[0, 0] == e and st.slot_of_expert[e] == loads[0, 1]
                assert cs[e] == -1
            assert int(st.tick[0]) == step + 1


def pin_cache_worked_example(lib):
    """Six experts, three slots, worked by hand from the policy's definition (misses by token count,
    ties to the lower expert; empty slots first, then least recently used, ties to the lower slot;
    slots of demanded experts are kept; this step computes only with experts already resident)."""
    st = oracle.CacheState(6, 3)
    steps = [
        # counts, max_loads, loads, compute_slot, slot_of_expert, expert_of_slot, last_use
        ([0, 3, 0, 3, 1, 0], 2, [(1, 0), (3, 1)], [-1] * 6, [-1, 0, -1, 1, -1, -1], [1, 3, -1], [1, 1, 0]),
        ([2, 0, 0, 1, 5, 0], 2, [(4, 2), (0, 0)], [-1, -1, -1, 1, -1, -1], [0, -1, -1, 1, 2, -1], [0, 3, 4],
         [2, 2, 2]),
        ([0, 1, 1, 0, 0, 1], 2, [(1, 0), (2, 1)], [-1, -1, -1, -1, 2, -1], [-1, 0, 1, -1, 2, -1], [1, 2, 4],
         [3, 3, 2]),
        ([0, 4, 0, 0, 0, 2], 2, [(5, 2)], [-1, 0, 1, -1, -1, -1], [-1, 0, 1, -1, -1, 2], [1, 2, 5], [4, 3, 4]),
        ([1, 1, 1, 1, 0, 1], 2, [], [-1, 0, 1, -1, -1, 2], [-1, 0, 1, -1, -1, 2], [1, 2, 5], [5, 5, 5]),
        ([0, 0, 0, 0, 0, 0], 2, [], [-1, 0, 1, -1, -1, 2], [-1, 0, 1, -1, -1, 2], [1, 2, 5], [5, 5, 5]),
        ([7, 0, 0, 0, 0, 0], 0, [], [-1, 0, 1, -1, -1, 2], [-1, 0, 1, -1, -1, 2], [1, 2, 5], [5, 5, 5]),
    ]
    for i, (counts, ml, loads, cs, soe, eos, lu) in enumerate(steps):
        got_cs, got_loads = oracle.cache_update(np.array(counts, np.int32), st, ml, lib=lib)
        assert [tuple(int(v) for v in r) for r in got_loads] == loads, (i, got_loads)
        assert got_cs.tolist() == cs, (i, got_cs)
        assert st.slot_of_expert.tolist() == soe and st.expert_of_slot.tolist() == eos, i
        assert st.last_use.tolist() == lu and int(st.tick[0]) == i + 1, i


def pin_cache_load_fraction(lib):
    """The load fraction caps the loads at ceil(q * m) of the m demanded absent experts (fp32 product),
    and load_slot names exactly this step's loads; worked by hand from the policy's definition."""
    st = oracle.CacheState(6, 4)
    steps = [
        # counts, max_loads, q, loads, compute_slot, load_slot
        ([1, 1, 1, 0, 0, 0], 4, 0.5, [(0, 0), (1, 1)], [-1] * 6, [0, 1, -1, -1, -1, -1]),
        ([0, 0, 3, 2, 0, 1], 4, 0.2, [(2, 2)], [0, 1, -1, -1, -1, -1], [-1, -1, 2, -1, -1, -1]),
        ([2, 0, 0, 1, 1, 0], 4, 1.0, [(3, 3), (4, 1)], [0, -1, 2, -1, -1, -1], [-1, -1, -1, 3, 1, -1]),
        ([0, 0, 0, 0, 0, 5], 4, 0.0, [(5, 2)], [0, -1, -1, 3, 1, -1], [-1, -1, -1, -1, -1, 2]),
    ]
    for i, (counts, ml, q, loads, cs, ls) in enumerate(steps):
        got_cs, got_loads, got_ls = oracle.cache_update(np.array(counts, np.int32), st, ml, q, lib=lib,
                                                        with_load_slot=True)
        assert [tuple(int(v) for v in r) for r in got_loads] == loads, (i, got_loads)
        assert got_cs.tolist() == cs and got_ls.tolist() == ls, (i, got_cs, got_ls)
    rng = np.random.default_rng(33)
    for q in (0.1, 0.37, 0.5, 0.9):
        st = oracle.CacheState(64, 24)
        pop = rng.permutation(64)
        for step in range(30):
            counts = np.bincount(_zipf_ids(rng, 6, 64, 4, pop).reshape(-1), minlength=64).astype(np.int32)
            prev = st.copy()
            cs, loads, ls = oracle.cache_update(counts, st, 24, q, lib=lib, with_load_slot=True)
            m = int(((counts > 0) & (prev.slot_of_expert < 0)).sum())
            idle = sum(1 for sl in range(24) if prev.expert_of_slot[sl] < 0 or counts[prev.expert_of_slot[sl]] == 0)
            share = int(np.ceil(np.float32(q) * np.float32(m)))
            assert len(loads) == min(m, idle, share), (q, step)
            want = np.full(64, -1, np.int32)
            for e, sl in loads:
                want[e] = sl
            assert np.array_equal(ls, want)


def _zipf_ids(rng, T, E, k, pop):
    p = 1.0 / np.arange(1, E + 1)
    p /= p.sum()
    return np.stack([pop[rng.choice(E, size=k, replace=False, p=p)] for _ in range(T)]).astype(np.int32)


def pin_cache_invariants(lib):
    """Random Zipf-skewed steps: the tables stay a bijection, demanded resident experts keep their
    slots, the loads are the misses with the most tokens put into the empty, then least recently
    used, slots whose experts are idle, and as many as the step allows."""
    rng = np.random.default_rng(32)
    for E, S, T, k, max_loads, steps in ((64, 16, 4, 4, 3, 80), (32, 32, 8, 2, 32, 40), (20, 6, 3, 3, 6, 60),
                                         (128, 96, 16, 8, 8, 40)):
        st = oracle.CacheState(E, S)
        pop = rng.permutation(E)
        for step in range(steps):
            counts = np.bincount(_zipf_ids(rng, T, E, k, pop).reshape(-1), minlength=E).astype(np.int32)
            prev = st.copy()
            cs, loads = oracle.cache_update(counts, st, max_loads, lib=lib)
            dem = counts > 0
            for sl in range(S):
                if st.expert_of_slot[sl] >= 0:
                    assert st.slot_of_expert[st.expert_of_slot[sl]] == sl
            assert (st.slot_of_expert >= 0).sum() == (st.expert_of_slot >= 0).sum()
            keep = dem & (prev.slot_of_expert >= 0)
            assert (st.slot_of_expert[keep] == prev.slot_of_expert[keep]).all()
            misses = [e for e in range(E) if dem[e] and prev.slot_of_expert[e] < 0]
            idle = [sl for sl in range(S) if prev.expert_of_slot[sl] < 0 or not dem[prev.expert_of_slot[sl]]]
            n = min(len(misses), max_loads, len(idle))
            assert len(loads) == n
            assert loads[:, 0].tolist() == sorted(misses, key=lambda e: (-counts[e], e))[:n]
            order = sorted(idle, key=lambda sl: (bool(prev.expert_of_slot[sl] >= 0), int(prev.last_use[sl]), sl))
            assert loads[:, 1].tolist() == order[:n]
            for e in range(E):
                same = prev.slot_of_expert[e] >= 0 and st.slot_of_expert[e] == prev.slot_of_expert[e]
                assert cs[e] == (prev.slot_of_expert[e] if same else -1)
            for e, sl in loads:
                assert st.slot_of_expert[e] == sl and st.last_use[sl] == step + 1
            for sl in range(S):
                v = st.expert_of_slot[sl]
                if v >= 0 and dem[v]:
                    assert st.last_use[sl] == step + 1
            assert int(st.tick[0]) == step + 1


ALL_PINS = [pin_route_bruteforce, pin_route_special_cases, pin_route_weights_float64, pin_permute,
            pin_decoder_tables, pin_dequant_roundtrip, pin_dequant_layouts, pin_ffn_float64,
            pin_layer_identical_experts, pin_layer_float64, pin_layer_sampled_threaded, pin_combine_cases, pin_router_logits_worked_example,
            pin_router_logits_one_hot, pin_router_logits_exact_sum, pin_cache_textbook_lru,
            pin_cache_worked_example, pin_cache_invariants, pin_cache_load_fraction]
