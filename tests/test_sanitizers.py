"""The CPU code under sanitizers (host compiler only; no GPU code is built here).

- The scalar C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (errors abort)
  runs every pin in a child process that preloads the sanitizer runtimes.
- The host residual routine (residual_host.cpp, threaded, with an atomic work counter) is built into
  a small driver with AddressSanitizer + UndefinedBehaviorSanitizer, and again with
  ThreadSanitizer, and run on hand-laid bf16 and FP8-B128 banks; its output must equal what the
  library's own build of the same routine gives on the same inputs (within fp32 contraction
  differences between the two builds).
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_wave_amd as ft
from host_banks import bf16_bank, fp8_bank

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
RESIDUAL_SRC = os.path.join(ROOT, "routed_expert_ffn_wave_amd", "csrc", "residual_host.cpp")
DRIVER_SRC = os.path.join(HERE, "sanitize", "residual_main.cpp")
ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "TSAN_OPTIONS": "halt_on_error=1"}


def _runtime(name: str) -> str:
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True).stdout.strip()


def _clean(r: subprocess.CompletedProcess):
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer"):
        assert marker not in text, text[-4000:]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "libftoracle_san.so")
    oracle.build(extra_flags=tuple(ASAN_UBSAN), out=so)
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle\n"
            "from oracle_pins import ALL_PINS\n"
            "lib = oracle._load(%r)\n"
            "for pin in ALL_PINS:\n"
            "    pin(lib)\n"
            "    print('ok', pin.__name__, flush=True)\n") % (ROOT, HERE, so)
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=f"{_runtime('libasan.so')}:{_runtime('libubsan.so')}")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    _clean(r)
    from oracle_pins import ALL_PINS
    assert r.stdout.count("ok ") == len(ALL_PINS)


def _build_driver(tmp_path, flags, name):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-O1", "-pthread", *flags, RESIDUAL_SRC, DRIVER_SRC, "-o", exe], check=True)
    return exe


def _cases():
    rng = np.random.default_rng(31)
    table = np.array([oracle.e4m3_value(int(c)) for c in range(256)], np.float32)
    T, k = 7, 3
    out = []
    for name, (hb, E, d, I) in (("bf16", (bf16_bank(rng, 5, 128, 64)[0], 5, 128, 64)),
                                ("fp8", (fp8_bank(rng, 4, 256, 128, table)[0], 4, 256, 128))):
        x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
        ids = torch.from_numpy(np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32))
        ids[1, 2] = E + 3                                   # an id outside the bank: never taken
        wts = torch.from_numpy(rng.random((T, k)).astype(np.float32))
        mask = torch.from_numpy(rng.integers(0, 1 << k, size=T).astype(np.int32))
        slots = torch.from_numpy(np.where(rng.random(E) < 0.5, -1, 0).astype(np.int32))
        out.append((name, hb, x, ids, wts, mask, slots))
    return out


def _write_case(d: str, hb, x, ids, wts, mask, slots, threads: int, use_mask: bool):
    os.makedirs(d, exist_ok=True)
    T, k = ids.shape
    with open(os.path.join(d, "params.txt"), "w") as f:
        f.write(f"{hb.fmt} {hb.n_slots} {hb.d} {hb.I} {T} {hb.n_slots} {k} {threads} {int(use_mask)} {int(not use_mask)}\n")
    arrays = {"w13": hb.w13, "w2": hb.w2, "s13": hb.s13, "s2": hb.s2, "x": x.view(torch.int16), "ids": ids, "w": wts,
              "mask": mask, "slots": slots}
    for key, t in arrays.items():
        if t is not None:
            t.contiguous().numpy().tofile(os.path.join(d, key + ".bin"))


@pytest.mark.parametrize("san", ["asan_ubsan", "tsan"])
def test_host_residual_under_sanitizers(tmp_path, san):
    # the thread sanitizer's runtime cannot start beside load-time resolvers of function clones, so its
    # build takes one baseline version of each loop
    flags = ASAN_UBSAN if san == "asan_ubsan" else ["-fsanitize=thread", "-g", "-DFT_HOST_CLONES="]
    exe = _build_driver(tmp_path, flags, f"residual_{san}")
    for name, hb, x, ids, wts, mask, slots in _cases():
        for threads in (1, 4):
            for use_mask in (True, False):
                d = str(tmp_path / f"{name}_{threads}_{int(use_mask)}")
                _write_case(d, hb, x, ids, wts, mask, slots, threads, use_mask)
                r = subprocess.run([exe, d], capture_output=True, text=True, env=dict(os.environ, **SAN_ENV),
                                   timeout=300)
                _clean(r)
                got = np.fromfile(os.path.join(d, "out.bin"), np.float32).reshape(x.shape[0], hb.d)
                ref = ft.ft_moe_residual_host(hb, x, ids, wts, mask if use_mask else None, n_threads=threads,
                                              slot_of_expert=None if use_mask else slots).numpy()
                assert int(r.stdout.strip()) >= 0
                scale = max(np.abs(ref).max(), 1e-30)
                assert np.abs(got - ref).max() <= 1e-5 * scale, (name, threads, use_mask)
