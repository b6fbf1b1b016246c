"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is the oracle source with one plausible mistake (a transposed operand,
a sign, a dropped term, an ignored weight, an unstable order, a wrong count),
built on the CPU into a temporary library.  The pin tests of the FFN, grouping,
union and bytes are then run against it; at least one must fail.  This shows
the pins constrain every part of the oracle, not only that the oracle agrees
with itself.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import ffn as oracle_ffn

from . import test_oracle_ffn as T_ffn
from . import test_oracle_group as T_grp
from . import test_oracle_union as T_uni

SRC = os.path.join(os.path.dirname(oracle_ffn.__file__), "moe_oracle.c")

MUTANTS = {
    "down_transposed": ("elem(wd, wdtype, (int64_t)i * d_ff + f)", "elem(wd, wdtype, (int64_t)f * d + i)"),
    "silu_sign": ("h[f] = a / (1.0 + exp(-a)) * b;", "h[f] = a / (1.0 + exp(a)) * b;"),
    "up_dropped": ("h[f] = a / (1.0 + exp(-a)) * b;", "h[f] = a / (1.0 + exp(-a));"),
    "gate_up_swapped": ("h[f] = a / (1.0 + exp(-a)) * b;", "h[f] = b / (1.0 + exp(-b)) * a;"),
    "weight_ignored": ("acc[(int64_t)t * d + i] += wt * o[i];", "acc[(int64_t)t * d + i] += o[i];"),
    "gate_row_stride": ("a += elem(wg, wdtype, (int64_t)f * d + i) * xi;",
                        "a += elem(wg, wdtype, (int64_t)i * d_ff + f) * xi;"),
    "unstable_scatter": ("for (int32_t s = 0; s < nm; ++s) {\n        if (!slot_valid(ids, m, N, s)) continue;\n        slot_by_expert[cursor[ids[s]]++] = s;",
                         "for (int32_t s = nm - 1; s >= 0; --s) {\n        if (!slot_valid(ids, m, N, s)) continue;\n        slot_by_expert[cursor[ids[s]]++] = s;"),
    "union_counts_repeats": ("        if (!seen[e]) {\n            seen[e] = 1;\n            ++u;\n        }",
                             "        seen[e] = 1;\n        ++u;"),
    "dedup_bytes_as_slot": ("if (kind == 1) return (int64_t)oracle_union_count(ids, n, m, N) * w;",
                            "if (kind == 1) return (int64_t)n * m * w;"),
    "duplicate_check_skipped": ("for (int32_t jj = 0; jj < j; ++jj)", "for (int32_t jj = 0; jj < 0; ++jj)"),
}

PINS = [
    lambda: T_ffn.test_single_expert_is_swiglu_mlp("bf16", 64, 96),
    lambda: T_ffn.test_single_expert_is_swiglu_mlp("f32", 40, 24),
    T_ffn.test_mixture_matches_torch_weighted_sum,
    T_ffn.test_identity_weights_closed_form,
    T_ffn.test_linear_in_routing_weights,
    T_ffn.test_invalid_ids_rejected,
    T_grp.test_grouping_brute_force_all_valid_arrays,
    T_grp.test_grouping_invalid_ids,
    T_grp.test_bytes_closed_forms,
    T_uni.test_exact_enumeration_tiny_mean_union,
]


def _build_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site of %s not unique in the oracle source" % name
    path_c = os.path.join(tmpdir, name + ".c")
    path_so = os.path.join(tmpdir, "lib" + name + ".so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", path_c, "-o", path_so, "-lm"])
    return path_so


def test_unmutated_copy_passes_pins():
    with tempfile.TemporaryDirectory() as td:
        so = os.path.join(td, "libcopy.so")
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", SRC, "-o", so, "-lm"])
        with oracle_ffn.use_library(so):
            for pin in PINS:
                pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    with tempfile.TemporaryDirectory() as td:
        so = _build_mutant(name, td)
        failures = 0
        with oracle_ffn.use_library(so):
            for pin in PINS:
                try:
                    pin()
                except (AssertionError, ValueError, pytest.fail.Exception):
                    failures += 1
        assert failures >= 1, "no pin caught the planted mistake %s" % name
    assert oracle.union_count([[0, 1]], 2) == 2  # the real oracle is back in place
