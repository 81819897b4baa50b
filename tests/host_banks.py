"""Expert banks laid out by hand in the library's documented device layout, in host memory, for the
CPU tests of the host residual path: 16-byte code chunks interleaved in blocks of 64 rows (chunk c
of row r at ((r/64 * nchunk + c) * 64 + r%64) * 16 bytes), W13 device block b = gate rows 32b..32b+31
then the matching up rows."""
from __future__ import annotations

import numpy as np
import torch

import routed_expert_ffn_wave_amd as ft


def _device_row(L: int, perm_I: int) -> int:
    """Device row of logical row L of a slot (W13 when perm_I > 0)."""
    if not perm_I:
        return L
    if L < perm_I:
        return 64 * (L >> 5) + (L & 31)
    return 64 * ((L - perm_I) >> 5) + 32 + ((L - perm_I) & 31)


def interleave(codes: np.ndarray, elem_bytes: int, perm_I: int) -> np.ndarray:
    """[E][R][K] codes of elem_bytes bytes each -> the interleaved byte array of all slots."""
    Em, R, K = codes.shape
    raw = np.ascontiguousarray(codes).view(np.uint8).reshape(Em * R, K * elem_bytes)
    nch = K * elem_bytes // 16
    out = np.zeros(Em * R * K * elem_bytes, np.uint8)
    for g in range(Em * R):
        slot, L = divmod(g, R)
        G = slot * R + _device_row(L, perm_I)
        for c in range(nch):
            off = (((G >> 6) * nch + c) * 64 + (G & 63)) * 16
            out[off:off + 16] = raw[g, 16 * c:16 * c + 16]
    return out


def bf16_bank(rng, E: int, d: int, I: int):
    """(host DeviceBank, fp32 W13 [E][2I][d], fp32 W2 [E][d][I]) of N(0, 0.05) weights rounded to bf16."""
    w13 = torch.from_numpy((rng.standard_normal((E, 2 * I, d)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    w2 = torch.from_numpy((rng.standard_normal((E, d, I)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    a13 = interleave(w13.view(torch.int16).numpy(), 2, I)
    a2 = interleave(w2.view(torch.int16).numpy(), 2, 0)
    hb = ft.DeviceBank(ft.FT_W_BF16, E, d, I, torch.from_numpy(a13), torch.from_numpy(a2))
    return hb, w13.float().numpy(), w2.float().numpy()


def fp8_bank(rng, E: int, d: int, I: int, e4m3_table: np.ndarray):
    """(host DeviceBank, fp32 W13, fp32 W2) of FP8-B128 codes covering every finite e4m3 byte, with
    fp32 scales per 128 x 128 block of logical rows; values from the given e4m3 decode table."""
    finite = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], np.uint8)

    def make(R, K, perm_I):
        codes = finite[rng.integers(0, len(finite), size=(E, R, K))]
        scales = (2.0 ** rng.integers(-12, -6, size=(E, R // 128, K // 128))).astype(np.float32)
        vals = e4m3_table[codes] * np.repeat(np.repeat(scales, 128, axis=1), 128, axis=2)
        return torch.from_numpy(interleave(codes, 1, perm_I)), torch.from_numpy(scales.reshape(-1).copy()), \
            vals.astype(np.float32)

    c13, s13, v13 = make(2 * I, d, I)
    c2, s2, v2 = make(d, I, 0)
    hb = ft.DeviceBank(ft.FT_W_FP8_B128, E, d, I, c13, c2, s13.view(torch.uint8), s2.view(torch.uint8))
    return hb, v13, v2
