"""The pins must catch plausible mistakes in the oracle (CPU only).

Each case compiles a copy of oracle/einsum_ref.c with one planted mistake (a
wrong sign, a dropped term, a transposed operand, a swapped aggregate, a
missing scale) into a temporary library, points the oracle at it, and checks
that at least one pin of test_oracle_definition fails.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle.ref as ref
from tests import test_oracle_definition as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "einsum_ref.c")

MUTATIONS = {
    "sqdiff_sign": ("case OR_JOIN_SQDIFF: return (x - y) * (x - y);",
                    "case OR_JOIN_SQDIFF: return (x + y) * (x + y);"),
    "dropped_last_term": ("if (++idx[cl[p]] < bounds[cl[p]])",
                          "if (++idx[cl[p]] < bounds[cl[p]] - 1)"),
    "transposed_operand": ("for (int p = n - 1; p >= 0; --p) {\n        st[p] = s;",
                           "for (int p = 0; p < n; ++p) {\n        st[p] = s;"),
    "max_is_min": ("else if (agg == OR_AGG_MAX) acc = v > acc ? v : acc;\n                else acc = v < acc ? v : acc;\n            } while (next_tuple(nc, cl, bounds, idx));\n            r = acc;\n        }\n        z[o] = post_scale * r;",
                   "else if (agg == OR_AGG_MAX) acc = v < acc ? v : acc;\n                else acc = v < acc ? v : acc;\n            } while (next_tuple(nc, cl, bounds, idx));\n            r = acc;\n        }\n        z[o] = post_scale * r;"),
    "scale_dropped": ("z[o] = post_scale * r;", "z[o] = r;"),
    "lse_without_max": ("r = m + log(s);", "r = log(s);"),
    "sub_operands_swapped": ("case OR_JOIN_SUB: return x - y;\n    }\n    return NAN;",
                             "case OR_JOIN_SUB: return y - x;\n    }\n    return NAN;"),
    "int_add_is_sub": ("static int64_t join_i(int op, int64_t x, int64_t y)\n{\n    switch (op) {\n    case OR_JOIN_MUL: return x * y;\n    case OR_JOIN_SQDIFF: return (x - y) * (x - y);\n    case OR_JOIN_ADD: return x + y;",
                       "static int64_t join_i(int op, int64_t x, int64_t y)\n{\n    switch (op) {\n    case OR_JOIN_MUL: return x * y;\n    case OR_JOIN_SQDIFF: return (x - y) * (x - y);\n    case OR_JOIN_ADD: return x - y;"),
}

PIN_FUNCS = [
    pins.test_hand_cases,
    pins.test_matmul_equals_library_product,
    pins.test_four_index_contraction_equals_library,
    pins.test_squared_distance_closed_form,
    pins.test_max_plus_special_cases,
    pins.test_logsumexp_closed_forms,
    pins.test_sub_join_closed_forms,
    pins.test_batched_and_attention_specs_equal_library,
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert old in src, f"mutation {name} no longer applies"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-fopenmp", "-o", str(lib), str(path), "-lm"], check=True)
    ref._load()  # make sure the real library's signatures are set up first
    mut = ctypes.CDLL(str(lib))
    for fn in ("oracle_einsum_f64", "oracle_einsum_i64"):
        getattr(mut, fn).argtypes = getattr(ref._lib, fn).argtypes
        getattr(mut, fn).restype = ctypes.c_int
    mut.oracle_max_threads.restype = ctypes.c_int
    monkeypatch.setattr(ref, "_lib", mut)
    caught = []
    for f in PIN_FUNCS:
        try:
            f()
        except AssertionError:
            caught.append(f.__name__)
    assert caught, f"no pin caught the planted mistake {name}"


# Planted mistakes in the oracle's cost model (oracle/chooser.py).  A mutated
# copy of the module is loaded in place of the real one, and the cost pins of
# test_oracle_chooser must fail against it.
CHOOSER_SRC = os.path.join(os.path.dirname(SRC), "chooser.py")
CHOOSER_MUTATIONS = {
    "softmax_drops_normalisation": ("        return lse + nrm\n", "        return lse\n"),
    "softmax_lse_over_s": ('lse = einsum_cost(f"{h}{s}{t}->{h}{s}"', 'lse = einsum_cost(f"{h}{s}{t}->{h}{t}"'),
    "softmax_broadcast_row_dropped": ('nrm = einsum_cost(f"{h}{s}{t},{h}{s}->{h}{s}{t}"',
                                      'nrm = einsum_cost(f"{h}{s}{t}->{h}{s}{t}"'),
    "aggregation_term_dropped": ("    return join_in + agg\n", "    return join_in\n"),
    "join_term_counts_groups": ("    join_in = n * sum(blk(o) for o in ops)",
                                "    join_in = (n // n_agg) * sum(blk(o) for o in ops)"),
}


@pytest.mark.parametrize("name", sorted(CHOOSER_MUTATIONS))
def test_planted_cost_model_mistake_is_caught(name, monkeypatch):
    import importlib.util
    import sys

    from tests import test_oracle_chooser as cpins
    old, new = CHOOSER_MUTATIONS[name]
    src = open(CHOOSER_SRC).read()
    assert old in src, f"mutation {name} no longer applies"
    spec = importlib.util.spec_from_loader("oracle._chooser_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = "oracle"
    monkeypatch.setitem(sys.modules, "oracle._chooser_mutant", mod)
    exec(compile(src.replace(old, new, 1), CHOOSER_SRC, "exec"), mod.__dict__)
    monkeypatch.setattr(cpins, "chooser", mod)
    caught = []
    for f in (cpins.test_hand_worked_costs, cpins.test_hand_worked_softmax_node_costs,
              cpins.test_softmax_node_best_blocking_closed_form):
        try:
            f()
        except AssertionError:
            caught.append(f.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
