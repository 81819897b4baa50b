"""Seeded synthetic inputs for one Mixture-of-Experts layer.

This module draws and encodes inputs only.  It holds none of the layer's
arithmetic (no routing, no dequantisation, no FFN): it is shared by the CPU
oracle and the HIP path so that both see the same bytes, and nothing else is.

Workloads are six MoE-layer shapes, with their sizes written out below.
The expert-bank formats are the ones the FreeToken
architecture walk-through lists for its expert banks ("深入FreeToken架构…全链路
剖析", section 五 "MoE 引擎": BF16 / FP8 block / NVFP4 / MXFP4 / GGUF Q4_0 each with its
own bank schema).  Encodings follow the public format definitions:

* Q4_0 (GGUF): blocks of 32 weights along K, 18 bytes each: an fp16 scale
  (little endian) then 16 bytes; byte i holds element i in its low nibble and
  element i+16 in its high nibble; value = scale * (q - 8).
* MXFP4 (OCP Microscaling v1.0): e2m1 elements, element 2i in the low nibble
  of byte i and 2i+1 in the high nibble; one E8M0 scale byte per 32 elements
  along K, stored in a separate [rows][K/32] array.
* FP8-B128: OCP e4m3fn elements with one fp32 scale per 128x128 block of
  (output row, K), stored as [rows/128][K/128].
* NVFP4: e2m1 elements packed as for MXFP4, one e4m3fn scale byte per 16
  elements along K ([rows][K/16]) and one fp32 scale for the whole matrix,
  stored after the block scales; value = tensor scale * e2m1 * e4m3.
* BF16: plain bf16, row-major.

Random numbers: each tensor has its own torch generator seeded from
numpy's SeedSequence([workload id, layer, stream, index]).  Streams:
0 logits, 1 activations, 2 popularity ranks, 3 slot table, 4/5/6 gate/up/down
weights (index = expert; the shared expert uses index E), 7 router rows.  The same seed gives
the same values on the same device type; CPU and GPU generators differ, which
is harmless because each parity check hands one set of tensors to both sides.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

FMT_BF16, FMT_Q4_0, FMT_MXFP4, FMT_FP8_B128, FMT_NVFP4 = 0, 1, 2, 3, 4
FMT_NAMES = {FMT_BF16: "bf16", FMT_Q4_0: "q4_0", FMT_MXFP4: "mxfp4", FMT_FP8_B128: "fp8_b128",
             FMT_NVFP4: "nvfp4"}

STREAM_LOGITS, STREAM_X, STREAM_RANK, STREAM_SLOTS, STREAM_GATE, STREAM_UP, STREAM_DOWN, STREAM_ROUTER = range(8)

WEIGHT_STD = 0.02
ZIPF_S = 1.1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One MoE-layer shape and its input recipe."""
    name: str
    wid: int            # workload id, first word of every seed
    T: int              # tokens (largest T of a sweep)
    d: int              # hidden size
    E: int              # routed experts
    k: int              # experts per token
    I: int              # expert intermediate size
    fmt: int            # bank format
    layers: int = 1     # independent layers run back to back
    zipf: bool = False  # per-expert popularity bias on the logits
    n_resident: int | None = None   # experts resident in the bank (None: all, identity table)
    shared: bool = False            # one always-on shared expert in bank slot E
    t_sweep: tuple = ()

    @property
    def n_slots(self) -> int:
        n = self.E if self.n_resident is None else self.n_resident
        return n + (1 if self.shared else 0)

    @property
    def shared_slot(self) -> int:
        return self.E if self.shared else -1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny layer: T=16, d=256, E=8, k=2, I=512, bf16 weights.
    "tiny_bf16": Workload("tiny_bf16", 0, T=16, d=256, E=8, k=2, I=512, fmt=FMT_BF16),
    # Decode, 35B-A3B-class shape, Q4_0 banks, 48 independent layers.
    "decode_q4_0": Workload("decode_q4_0", 1, T=8, d=2048, E=128, k=8, I=768, fmt=FMT_Q4_0, layers=48),
    # Prefill chunk of the same shape, bf16 banks, Zipf-skewed routing.
    "prefill_bf16_zipf": Workload("prefill_bf16_zipf", 2, T=4096, d=2048, E=128, k=8, I=768,
                                  fmt=FMT_BF16, zipf=True),
    # 284B-class layer, MXFP4 banks, 256 routed + 1 shared expert, T=16 and T=8192.
    "mxfp4_shared": Workload("mxfp4_shared", 3, T=8192, d=7168, E=256, k=8, I=2048, fmt=FMT_MXFP4,
                             shared=True, t_sweep=(16, 8192)),
    # Resident-bank layer: FP8-B128 banks, 96 of 256 experts resident, residual mask, T sweep.
    "fp8_resident": Workload("fp8_resident", 4, T=16384, d=7168, E=256, k=8, I=2048, fmt=FMT_FP8_B128,
                             zipf=True, n_resident=96, t_sweep=(1, 16, 256, 4096, 16384)),
    # The decode shape above with NVFP4 banks (the fifth bank format of the walk-through).
    "nvfp4_decode": Workload("nvfp4_decode", 5, T=8, d=2048, E=128, k=8, I=768, fmt=FMT_NVFP4, layers=48),
}


def seed_of(wid: int, layer: int, stream: int, index: int = 0) -> int:
    ss = np.random.SeedSequence([wid, layer, stream, index])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(device, wid, layer, stream, index=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(wid, layer, stream, index))
    return g


# --------------------------------------------------------------------------------------------
# activations, logits, slot table


def zipf_bias(w: Workload, layer: int) -> torch.Tensor:
    """Per-expert logit bias -s*ln(rank) from a seeded popularity ranking (rank 1 = most popular)."""
    g = _gen("cpu", w.wid, layer, STREAM_RANK)
    rank = torch.randperm(w.E, generator=g) + 1
    return (-ZIPF_S * torch.log(rank.double())).float()


def logits(w: Workload, layer: int = 0, T: int | None = None, device="cpu") -> torch.Tensor:
    """fp32 router logits [T][E]: N(0,1), plus the Zipf bias when the workload is skewed.

    A sweep over T uses the first T rows of the largest tensor."""
    T = w.T if T is None else T
    g = _gen(device, w.wid, layer, STREAM_LOGITS)
    L = torch.randn(w.T, w.E, generator=g, device=device, dtype=torch.float32)
    if w.zipf:
        L = L + zipf_bias(w, layer).to(device)
    return L[:T].contiguous()


def step_logits(w: Workload, step: int, T: int | None = None, device="cpu") -> torch.Tensor:
    """Router logits [T][E] of one step of a stream of steps: fresh N(0,1) per step plus one Zipf
    popularity bias for the whole stream (the first layer's), so popular experts recur."""
    T = w.T if T is None else T
    g = _gen(device, w.wid, 0, STREAM_LOGITS, 1 + step)
    L = torch.randn(T, w.E, generator=g, device=device, dtype=torch.float32)
    return (L + zipf_bias(w, 0).to(device)).contiguous()


def zipf_counts(E: int, T: int, k: int, seed: int, step: int) -> np.ndarray:
    """int32 [E] tokens per expert of one step: each of T tokens picks k distinct experts with
    probability proportional to 1/rank over a seeded popularity order (the same for every step)."""
    order = np.random.default_rng([seed, 0]).permutation(E)
    p = 1.0 / np.arange(1, E + 1)
    p /= p.sum()
    rng = np.random.default_rng([seed, 1 + step])
    ids = np.concatenate([order[rng.choice(E, size=k, replace=False, p=p)] for _ in range(T)])
    return np.bincount(ids, minlength=E).astype(np.int32)


def activations(w: Workload, layer: int = 0, T: int | None = None, device="cpu") -> torch.Tensor:
    """bf16 activations [T][d] drawn N(0,1) in fp32 and rounded to nearest even."""
    T = w.T if T is None else T
    g = _gen(device, w.wid, layer, STREAM_X)
    x = torch.randn(w.T, w.d, generator=g, device=device, dtype=torch.float32)
    return x[:T].to(torch.bfloat16).contiguous()


def router_rows(w: Workload, layer: int = 0, device="cpu") -> torch.Tensor:
    """bf16 router rows [E][d] drawn N(0, 1/d) in fp32 and rounded to nearest even, so that the
    router logits of N(0,1) activations are about N(0,1), like the workloads' logits."""
    g = _gen(device, w.wid, layer, STREAM_ROUTER)
    wr = torch.randn(w.E, w.d, generator=g, device=device, dtype=torch.float32) / float(np.sqrt(w.d))
    return wr.to(torch.bfloat16).contiguous()


def slot_table(w: Workload, layer: int = 0) -> torch.Tensor:
    """int32 expert -> bank slot map; -1 marks an expert that is not resident.

    Identity when every expert is resident; otherwise a random n_resident of the E experts
    placed in a shuffled slot order."""
    if w.n_resident is None:
        return torch.arange(w.E, dtype=torch.int32)
    g = _gen("cpu", w.wid, layer, STREAM_SLOTS)
    perm = torch.randperm(w.E, generator=g)
    table = torch.full((w.E,), -1, dtype=torch.int32)
    table[perm[: w.n_resident]] = torch.arange(w.n_resident, dtype=torch.int32)
    return table


def slot_experts(w: Workload, layer: int = 0) -> list[int]:
    """Expert index held by each bank slot (the shared expert is index E)."""
    table = slot_table(w, layer)
    n = w.E if w.n_resident is None else w.n_resident
    experts = [0] * n
    for e, s in enumerate(table.tolist()):
        if s >= 0:
            experts[s] = e
    if w.shared:
        experts.append(w.E)
    return experts


def expert_weights(w: Workload, layer: int, expert: int, device="cpu"):
    """fp32 weights of one expert before quantisation: W13 [2I][d] (gate rows, then up rows), W2 [d][I]."""
    gg = _gen(device, w.wid, layer, STREAM_GATE, expert)
    gu = _gen(device, w.wid, layer, STREAM_UP, expert)
    gd = _gen(device, w.wid, layer, STREAM_DOWN, expert)
    w13 = torch.empty(2 * w.I, w.d, device=device, dtype=torch.float32)
    w13[: w.I].normal_(0.0, WEIGHT_STD, generator=gg)
    w13[w.I:].normal_(0.0, WEIGHT_STD, generator=gu)
    w2 = torch.empty(w.d, w.I, device=device, dtype=torch.float32).normal_(0.0, WEIGHT_STD, generator=gd)
    return w13, w2


# --------------------------------------------------------------------------------------------
# encoders (fp32 weights -> stored bytes); inputs only


def encode_bf16(wt: torch.Tensor):
    return wt.to(torch.bfloat16).view(torch.int16), None


def encode_q4_0(wt: torch.Tensor):
    """GGUF Q4_0 blocks, [rows][K/32][18] uint8.

    scale = (the block's value of largest magnitude) / -8 stored as fp16;
    q = clamp(round_half_even(w / scale) + 8, 0, 15)."""
    rows, K = wt.shape
    assert K % 32 == 0
    b = wt.reshape(rows, K // 32, 32)
    idx = b.abs().argmax(dim=-1, keepdim=True)
    vmax = torch.gather(b, -1, idx)
    scale16 = (vmax / -8.0).to(torch.float16)
    s = scale16.float()
    inv = torch.where(s != 0, 1.0 / s, torch.zeros_like(s))
    q = (torch.round(b * inv) + 8.0).clamp(0, 15).to(torch.uint8)
    out = torch.empty(rows, K // 32, 18, dtype=torch.uint8, device=wt.device)
    out[..., 0:2] = scale16.view(torch.uint8).reshape(rows, K // 32, 2)
    out[..., 2:18] = q[..., :16] | (q[..., 16:] << 4)
    return out, None


_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def encode_mxfp4(wt: torch.Tensor):
    """OCP MXFP4: codes [rows][K/2] uint8 (element 2i low nibble), E8M0 scales [rows][K/32] uint8.

    Shared exponent = floor(log2(amax)) - 2 (2 = largest e2m1 exponent); elements are rounded
    to the nearest e2m1 value with ties to the even code and saturated at 6."""
    rows, K = wt.shape
    assert K % 32 == 0
    b = wt.reshape(rows, K // 32, 32)
    amax = b.abs().amax(dim=-1, keepdim=True)
    e = torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2.0
    e = torch.where(amax > 0, e, torch.full_like(e, -127.0)).clamp(-127, 127)
    v = b / torch.exp2(e)
    a = v.abs()
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=wt.device)
    dist = (a.unsqueeze(-1) - grid).abs()
    best = dist.amin(dim=-1, keepdim=True)
    codes = torch.arange(8, device=wt.device)
    score = (dist == best).to(torch.int32) * (2 - (codes & 1))
    mag = score.argmax(dim=-1).to(torch.uint8)
    sign = ((v < 0) & (mag != 0)).to(torch.uint8) << 3
    c = (mag | sign).reshape(rows, K)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).contiguous()
    scales = (e + 127).to(torch.uint8).reshape(rows, K // 32).contiguous()
    return packed, scales


def encode_fp8_b128(wt: torch.Tensor):
    """FP8 e4m3fn codes [rows][K] uint8 with fp32 scales [rows/128][K/128]; scale = block amax / 448."""
    rows, K = wt.shape
    assert rows % 128 == 0 and K % 128 == 0
    b = wt.reshape(rows // 128, 128, K // 128, 128)
    amax = b.abs().amax(dim=(1, 3), keepdim=True)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (b / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(rows, K).contiguous(), scale.reshape(rows // 128, K // 128).contiguous()


def _e2m1_codes(v: torch.Tensor) -> torch.Tensor:
    """Nearest e2m1 code of each value (ties to the even code), saturating at 6; sign in bit 3."""
    a = v.abs()
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float32, device=v.device)
    dist = (a.unsqueeze(-1) - grid).abs()
    best = dist.amin(dim=-1, keepdim=True)
    codes = torch.arange(8, device=v.device)
    score = (dist == best).to(torch.int32) * (2 - (codes & 1))
    mag = score.argmax(dim=-1).to(torch.uint8)
    return mag | (((v < 0) & (mag != 0)).to(torch.uint8) << 3)


def encode_nvfp4(wt: torch.Tensor):
    """NVFP4: codes [rows][K/2] uint8 (element 2i low nibble), scales uint8 [rows*K/16 + 4]: one
    e4m3fn scale per 16 elements along K, then the matrix's fp32 scale (4 bytes, little endian).

    tensor scale t = amax / (448 * 6), so that block scales fit e4m3; block scale
    s = e4m3(block amax / 6 / t) (round to nearest even, saturating at 448); elements are the
    nearest e2m1 values of w / (t * s) (ties to the even code, saturating at 6)."""
    rows, K = wt.shape
    assert K % 32 == 0
    amax = wt.abs().amax()
    t = (amax / (448.0 * 6.0)).float() if amax > 0 else torch.tensor(1.0, device=wt.device)
    b = wt.reshape(rows, K // 16, 16)
    bmax = b.abs().amax(dim=-1, keepdim=True)
    sq = (bmax / 6.0 / t).clamp(max=448.0).to(torch.float8_e4m3fn)
    s = sq.float()
    denom = torch.where(s > 0, s * t, torch.ones_like(s))
    v = torch.where(s > 0, b / denom, torch.zeros_like(b))
    c = _e2m1_codes(v).reshape(rows, K)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).contiguous()
    scales = torch.empty(rows * (K // 16) + 4, dtype=torch.uint8, device=wt.device)
    scales[: rows * (K // 16)] = sq.view(torch.uint8).reshape(-1)
    scales[rows * (K // 16):] = t.reshape(1).view(torch.uint8)
    return packed, scales


ENCODERS = {FMT_BF16: encode_bf16, FMT_Q4_0: encode_q4_0, FMT_MXFP4: encode_mxfp4,
            FMT_FP8_B128: encode_fp8_b128, FMT_NVFP4: encode_nvfp4}


def code_shape(fmt: int, rows: int, K: int):
    """Shape and dtype of the stored element codes of one [rows][K] matrix (canonical layout)."""
    if fmt == FMT_BF16:
        return (rows, K), torch.int16
    if fmt == FMT_Q4_0:
        return (rows, K // 32, 18), torch.uint8
    if fmt in (FMT_MXFP4, FMT_NVFP4):
        return (rows, K // 2), torch.uint8
    if fmt == FMT_FP8_B128:
        return (rows, K), torch.uint8
    raise ValueError(fmt)


def scale_shape(fmt: int, rows: int, K: int):
    if fmt == FMT_MXFP4:
        return (rows, K // 32), torch.uint8
    if fmt == FMT_FP8_B128:
        return (rows // 128, K // 128), torch.float32
    if fmt == FMT_NVFP4:
        return (rows * (K // 16) + 4,), torch.uint8
    return None, None


@dataclasses.dataclass
class Bank:
    """Canonical expert bank: per-slot stored codes and scales of W13 [2I][d] and W2 [d][I]."""
    fmt: int
    d: int
    I: int
    w13: torch.Tensor
    w2: torch.Tensor
    s13: torch.Tensor | None
    s2: torch.Tensor | None

    @property
    def n_slots(self) -> int:
        return self.w13.shape[0]

    def to(self, device) -> "Bank":
        f = lambda t: None if t is None else t.to(device)
        return Bank(self.fmt, self.d, self.I, f(self.w13), f(self.w2), f(self.s13), f(self.s2))

    def slot(self, s: int, device="cpu") -> "Bank":
        f = lambda t: None if t is None else t[s:s + 1].to(device)
        return Bank(self.fmt, self.d, self.I, f(self.w13), f(self.w2), f(self.s13), f(self.s2))


def empty_bank(fmt: int, n_slots: int, d: int, I: int, device="cpu") -> Bank:
    cs13, ct = code_shape(fmt, 2 * I, d)
    cs2, _ = code_shape(fmt, d, I)
    ss13, st = scale_shape(fmt, 2 * I, d)
    ss2, _ = scale_shape(fmt, d, I)
    w13 = torch.empty((n_slots,) + cs13, dtype=ct, device=device)
    w2 = torch.empty((n_slots,) + cs2, dtype=ct, device=device)
    s13 = None if ss13 is None else torch.empty((n_slots,) + ss13, dtype=st, device=device)
    s2 = None if ss2 is None else torch.empty((n_slots,) + ss2, dtype=st, device=device)
    return Bank(fmt, d, I, w13, w2, s13, s2)


def fill_slot(bank: Bank, slot: int, w13: torch.Tensor, w2: torch.Tensor) -> None:
    """Encode fp32 weights into one bank slot."""
    enc = ENCODERS[bank.fmt]
    c13, s13 = enc(w13)
    c2, s2 = enc(w2)
    bank.w13[slot].copy_(c13.reshape(bank.w13.shape[1:]))
    bank.w2[slot].copy_(c2.reshape(bank.w2.shape[1:]))
    if bank.s13 is not None:
        bank.s13[slot].copy_(s13)
        bank.s2[slot].copy_(s2)


def make_bank(w: Workload, layer: int = 0, device="cpu") -> Bank:
    """The workload's canonical bank: one slot per resident expert (slot order of the table),
    plus the shared expert in the last slot when the workload has one."""
    experts = slot_experts(w, layer)
    bank = empty_bank(w.fmt, len(experts), w.d, w.I, device=device)
    for s, e in enumerate(experts):
        w13, w2 = expert_weights(w, layer, e, device=device)
        fill_slot(bank, s, w13, w2)
    return bank


@dataclasses.dataclass
class LayerInputs:
    workload: Workload
    layer: int
    T: int
    logits: torch.Tensor      # fp32 [T][E]
    x: torch.Tensor           # bf16 [T][d]
    slot_of_expert: torch.Tensor  # int32 [E]
    bank: Bank


def layer_inputs(w: Workload, layer: int = 0, T: int | None = None, device="cpu") -> LayerInputs:
    T = w.T if T is None else T
    return LayerInputs(w, layer, T, logits(w, layer, T, device), activations(w, layer, T, device),
                       slot_table(w, layer).to(device), make_bank(w, layer, device))


def bytes_per_weight(fmt: int) -> float:
    """Stored bytes per weight including scales."""
    return {FMT_BF16: 2.0, FMT_Q4_0: 18.0 / 32.0, FMT_MXFP4: 17.0 / 32.0,
            FMT_FP8_B128: 1.0 + 4.0 / (128 * 128), FMT_NVFP4: 9.0 / 16.0}[fmt]


def expert_bytes(fmt: int, d: int, I: int) -> float:
    return 3.0 * d * I * bytes_per_weight(fmt)


def small(w: Workload, **kw) -> Workload:
    """Same recipe at other sizes (for tests that must finish in seconds on the CPU)."""
    return w.replace(**kw)


