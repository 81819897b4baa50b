"""Planted mistakes in the oracle must trip at least one pin.

Each case copies ftoracle.c, makes one plausible mistake (a dropped term, a wrong sign or index, a
swapped operand), builds it with the oracle's own flags and runs every pin against it.  This runs on
the CPU only; the planted copies live in a temporary directory.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "ftoracle.c")

MUTANTS = {
    "route_ties_to_highest": ("if (best < 0 || L[e] > L[best]) best = e;", "if (best < 0 || L[e] >= L[best]) best = e;"),
    "route_no_renormalise": ("wt[j] = (p[id[j]] / Z) / S;", "wt[j] = (p[id[j]] / Z);"),
    "route_softmax_sign": ("p[e] = expf(L[e] - m);", "p[e] = expf(m - L[e]);"),
    "permute_unstable": ("for (int f = 0; f < n; ++f)\n      if (ids[f] == e) {", "for (int f = n - 1; f >= 0; --f)\n      if (ids[f] == e) {"),
    "permute_inclusive_offsets": ("offsets[e + 1] = offsets[e] + counts[e];", "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);"),
    "permute_inv_dropped": ("inv[f] = pos;", "inv[f] = f;"),
    "fp16_bias": ("v = ldexpf((float)(1024 + m), e - 25);", "v = ldexpf((float)(1024 + m), e - 24);"),
    "e2m1_bias": ("ldexpf(1.0f + 0.5f * (float)m, e - 1)", "ldexpf(1.0f + 0.5f * (float)m, e)"),
    "e2m1_subnormal": ("0.5f * (float)m : ldexpf", "1.0f * (float)m : ldexpf"),
    "e4m3_subnormal": ("v = ldexpf((float)m, -9);", "v = ldexpf((float)m, -10);"),
    "e4m3_nan": ("if (e == 15 && m == 7)", "if (e == 15 && m == 8)"),
    "e8m0_bias": ("ldexpf(1.0f, (int)s - 127)", "ldexpf(1.0f, (int)s - 128)"),
    "q4_offset": ("o[32 * b + i] = scale * (float)(lo - 8);", "o[32 * b + i] = scale * (float)(lo - 7);"),
    "q4_nibble_order": ("o[32 * b + i + 16] = scale * (float)(hi - 8);", "o[32 * b + i + 16] = scale * (float)(lo - 8);"),
    "mx_nibble_order": ("unsigned q = (j & 1) ? (c[j / 2] >> 4) : (c[j / 2] & 15);", "unsigned q = (j & 1) ? (c[j / 2] & 15) : (c[j / 2] >> 4);"),
    "mx_scale_index": ("ora_e8m0_value(s[j / 32])", "ora_e8m0_value(s[j / 64])"),
    "nv_nibble_order": ("(c[j >> 1] >> (4 * (j & 1))) & 15u", "(c[j >> 1] >> (4 * (1 - (j & 1)))) & 15u"),
    "nv_scale_index": ("ora_e4m3_value(s[j / 16])", "ora_e4m3_value(s[j / 32])"),
    "nv_tensor_scale_dropped": ("o[j] = t * (ora_e2m1_value(q) * ora_e4m3_value(s[j / 16]));", "o[j] = ora_e2m1_value(q) * ora_e4m3_value(s[j / 16]);"),
    "fp8_block_row": ("(size_t)(r / 128) * (K / 128)", "(size_t)(r % 2) * (K / 128)"),
    "fp8_block_col": ("o[j] = s[j / 128] * ora_e4m3_value(c[j]);", "o[j] = s[0] * ora_e4m3_value(c[j]);"),
    "silu_sign": ("hr[i] = g / (1.0f + expf(-g)) * u;", "hr[i] = g / (1.0f + expf(g)) * u;"),
    "gate_up_swapped": ("const float* wg = w13 + (size_t)i * d;", "const float* wg = w13 + (size_t)(I + i) * d;"),
    "down_transposed": ("acc = acc + hr[i] * wd[i];", "acc = acc + hr[i] * w2[(size_t)i * d + c % d];"),
    "combine_no_weight": ("o[c] = o[c] + wj * yr[c];", "o[c] = o[c] + yr[c];"),
    "combine_no_shared": ("o[c] = o[c] + ys[c];", "o[c] = o[c];"),
    "mask_wrong_bit": ("bits |= 1u << j;", "bits |= 1u << (k - 1 - j);"),
    "router_transposed": ("(double)ora_bf16_value(wr[(size_t)e * d + c]);", "(double)ora_bf16_value(wr[((size_t)c * E + e) % ((size_t)E * d)]);"),
    "router_dropped_term": ("for (int c = 0; c < d; ++c)\n        acc +=", "for (int c = 1; c < d; ++c)\n        acc +="),
    "lru_evicts_mru": ("(occ == occ_best && last_use[s] < last_use[slot])", "(occ == occ_best && last_use[s] > last_use[slot])"),
    "lru_ties_to_highest_slot": ("last_use[s] < last_use[slot])) slot = s;", "last_use[s] <= last_use[slot])) slot = s;"),
    "lru_occupied_first": ("if (occ < occ_best ||", "if (occ > occ_best ||"),
    "lru_misses_by_index": ("(want < 0 || counts[e] > counts[want])", "(want < 0)"),
    "lru_evicts_demanded": ("if (v >= 0 && counts[v] > 0) continue;", "if (v >= 0 && counts[v] < 0) continue;"),
    "lru_no_refresh": ("last_use[slot_of_expert[e]] = now;", "last_use[slot_of_expert[e]] = last_use[slot_of_expert[e]];"),
    "lru_fraction_floor": ("const int share = (int)ceilf(load_fraction * (float)m);", "const int share = (int)floorf(load_fraction * (float)m);"),
    "lru_load_slot_all": ("load_slot[e] = (before[e] < 0 && slot_of_expert[e] >= 0) ? slot_of_expert[e] : -1;", "load_slot[e] = slot_of_expert[e];"),
    "lru_compute_with_loads": ("compute_slot[e] = (before[e] >= 0 && slot_of_expert[e] == before[e]) ? before[e] : -1;", "compute_slot[e] = slot_of_expert[e];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
    msrc = tmp_path / "ftoracle.c"
    msrc.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *[f for f in oracle.CFLAGS if f != "-Werror"], str(msrc), "-o", str(so), "-lm"], check=True)
    lib = oracle._load(str(so))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"


# Planted mistakes in the Python composition of the layer (oracle/__init__.py): the token filter,
# the threaded runs and the compaction of the computed rows.  Each must trip the pin of the
# sampled, threaded layer (or the other layer pins).
PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
PY_MUTANTS = {
    "filter_by_slot_index": ("pos = pos[want[gather[pos] // k]]", "pos = pos[want[gather[pos] % k]]"),
    "filter_dropped": ("pos = pos[want[gather[pos] // k]]", "pos = pos"),
    "threaded_runs_reordered": ("ys = list(ex.map(run, jobs))", "ys = list(ex.map(run, jobs))[::-1]"),
    "run_truncated": ("jobs.append((s, pos[r0:r0 + step]))", "jobs.append((s, pos[r0:r0 + step - 1]))"),
    "compaction_uses_sorted_row": ("local_inv[flat_ok] = local[inv[flat_ok]]", "local_inv[flat_ok] = inv[flat_ok]"),
    "shared_rows_unfiltered": ("_, ysh = swiglu_ffn(xf[tok], w13, w2, lib=lib)", "_, ysh = swiglu_ffn(xf[:len(tok)], w13, w2, lib=lib)"),
    "combine_all_tokens": ("tok_list = np.nonzero(want)[0].astype(np.int32)", "tok_list = np.arange(T, dtype=np.int32)"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_layer_mutant_is_caught(name, tmp_path):
    import importlib.util

    from oracle_pins import pin_layer_float64, pin_layer_identical_experts, pin_layer_sampled_threaded
    old, new = PY_MUTANTS[name]
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
    path = tmp_path / "oracle_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    lib = oracle._load()
    caught = []
    for pin in (pin_layer_sampled_threaded,):
        try:
            pin(lib, ora=mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed the layer pins"
    # the unplanted module passes the same pins (the planted copy differs only at the mutation site)
    for pin in (pin_layer_float64, pin_layer_identical_experts):
        pin(lib)
