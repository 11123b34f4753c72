"""Planted mistakes: each case copies oracle/k3oracle.c, injects one
plausible wrong implementation (a textual substitution), builds it on the CPU
and runs the pin checks against it. Every mutant must fail at least one pin;
otherwise the pins would not protect the oracle against that mistake.
The mistakes are those the pages warn about (nibble order, NaN scale, bias
leaking into the weights) plus common slips (exponent bias, table sign,
scale indexing, gate/up swap, missing renormalisation, tie order, rounding
ties)."""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import _pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "k3oracle.c")

MUTANTS = {
    "swapped_nibbles": ("return (j % 2 == 0) ? (byte & 15) : (byte >> 4);",
                        "return (j % 2 == 0) ? (byte >> 4) : (byte & 15);"),
    "e8m0_bias_128": ("return ldexp(1.0, e - 127);", "return ldexp(1.0, e - 128);"),
    "nan_scale_as_number": ("if (e == 255) continue; /* NaN scale: the group contributes nothing */",
                            "/* 255 used as a number */"),
    "code8_as_plus8": ("-0.0, -0.5, -1.0", "8.0, -0.5, -1.0"),
    "scale_per_element": ("sc[(size_t)r * (size_t)(cols / 32) + (size_t)(j / 32)]",
                          "sc[(size_t)r * (size_t)(cols / 32) + (size_t)(j % (cols / 32))]"),
    "silu_on_up": ("hh[i] = k3o_silu(g[i]) * u[i];", "hh[i] = g[i] * k3o_silu(u[i]);"),
    "bias_leaks_into_weights": ("w[j] = sigmoid(logits[idx[j]]);", "w[j] = key[idx[j]];"),
    "no_renormalisation": ("for (int j = 0; j < k; j++) w[j] = w[j] / sum;", "(void)sum;"),
    "ties_to_higher_index": ("if (best < 0 || key[e] > key[best]) best = e;",
                             "if (best < 0 || key[e] >= key[best]) best = e;"),
    "quant_ties_away": ("if (d < db || (d == db && (m % 2 == 0))) best = m;",
                        "if (d < db || d == db) best = m;"),
    "quant_scale_off_by_one": ("int E = (ex - 1) - 2;", "int E = (ex - 1) - 3;"),
    "router_drops_last_term": ("for (int k = 0; k < hidden; k++)\n      acc +=",
                               "for (int k = 0; k < hidden - 1; k++)\n      acc +="),
    "shared_gate_up_swapped": ("hh[i] = k3o_silu(g) * u;", "hh[i] = k3o_silu(u) * g;"),
    "shared_down_transposed": ("y[r] = dot_bf16_row(S->down + (size_t)r * inter, hh, inter);",
                               "{ y[r] = 0.0; for (int c = 0; c < inter; c++) y[r] += "
                               "k3o_bf16_to_f64(S->down[(size_t)c * hidden + r]) * hh[c]; }"),
    "shared_not_added": ("for (int r = 0; !rc && r < hidden; r++) y[r] += ys[r];",
                         "(void)ys;"),
    "combine_drops_rank0": ("for (int j = 0; j < k; j++) acc += w[j] * ye[(size_t)j * hidden + i];",
                            "for (int j = 1; j < k; j++) acc += w[j] * ye[(size_t)j * hidden + i];"),
    "bf16_ties_away": ("if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) r = hi + 1u;",
                       "if (lo >= 0x8000u) r = hi + 1u;"),
    "bf16_truncation": ("if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) r = hi + 1u;",
                        "(void)lo;"),
    "logits_offset_ignored": ("logits + (size_t)t * n_experts, bias, experts,",
                              "logits, bias, experts,"),
}


@pytest.fixture(scope="module")
def tmpdir_mod():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mod):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once for {name}"
    path_c = os.path.join(tmpdir_mod, f"m_{name}.c")
    path_so = os.path.join(tmpdir_mod, f"libm_{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    inc = os.path.dirname(SRC)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-I", inc,
                           path_c, "-o", path_so, "-lm"])
    O = oracle.Oracle(path_so)
    failed = []
    for check in P.ALL:
        try:
            check(O)
        except (AssertionError, oracle.OracleError, IndexError, ValueError):
            failed.append(check.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
