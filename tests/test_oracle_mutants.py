"""The oracle's pins catch plausible mistakes.

Each mutant below plants one mistake in a copy of the oracle's C source (a
dropped term, a wrong sign, a wrong operand or index, a tie rule flipped),
builds it into a temporary library and runs the CPU pins of test_oracle.py
against it: at least one pin must fail. The real oracle is restored after.
"""
import os
import subprocess
import tempfile

import pytest

from oracle import oracle as orc_mod
import test_oracle as pins

MUTANTS = {
    "gate drops last term": ("wg_t + (i64)i * dm, dm);\n}", "wg_t + (i64)i * dm, dm - 1);\n}"),
    "pack keeps g == 0": ("if (v > 0.0) {", "if (v >= 0.0) {"),
    "pack stores tile-local column": ("col[base + n] = c;", "col[base + n] = c - j * tile_c;"),
    "sparse fwd drops up projection": ("double a = val[e] * u;", "double a = val[e];"),
    "dense fwd uses gate weights for up": ("double u = dot(xt, wu_t + (i64)i * dm, dm);\n            double a = h * u;",
                                           "double u = dot(xt, wg_t + (i64)i * dm, dm);\n            double a = h * u;"),
    "hybrid tie goes to backup": ("if (nnz <= K) {", "if (nnz < K) {"),
    "hybrid backup row id": ("ovf_rows[n] = t;", "ovf_rows[n] = n;"),
    "bwd dg uses h": ("cdg[e] = da * u + l1;", "cdg[e] = da * r.h[e] + l1;"),
    "bwd drops the L1 term": ("cdg[e] = da * u + l1;", "cdg[e] = da * u;"),
    "bwd L1 term weighted by h": ("cdg[e] = da * u + l1;", "cdg[e] = da * u + l1 * r.h[e];"),
    "bwd da from up weights": ("double da = dot(dyt, wd + (i64)i * dm, dm);\n                ca[e]",
                               "double da = dot(dyt, wu_t + (i64)i * dm, dm);\n                ca[e]"),
    "hybrid fwd drops up projection": ("double a = r.h[e] * dot(xt, wu_t + (i64)i * dm, dm);",
                                       "double a = r.h[e];"),
    "hybrid fwd down row from up weights": ("const double *wdi = wd + (i64)i * dm;\n            for (int k = 0; k < dm; ++k)\n                yt[k] += a * wdi[k];\n        }\n    }\n    free(r.off);",
                                            "const double *wdi = wu_t + (i64)i * dm;\n            for (int k = 0; k < dm; ++k)\n                yt[k] += a * wdi[k];\n        }\n    }\n    free(r.off);"),
    "bwd dx sign": ("dxt[k] = su[k] + sg[k];", "dxt[k] = su[k] - sg[k];"),
    "bwd dW_u from dy": ("dwu_t[o + k] += cdu[e] * xt[k];", "dwu_t[o + k] += cdu[e] * dyt[k];"),
    "bwd dW_d from x": ("dwd[o + k] += ca[e] * dyt[k];", "dwd[o + k] += ca[e] * xt[k];"),
    "bwd drops dg term of dx": ("sg[k] += cdg[e] * wgi[k];", "sg[k] += 0.0 * wgi[k];"),
}

PIN_FUNCS = [
    lambda o: pins.test_worked_example_forward(o),
    lambda o: pins.test_worked_example_hybrid_and_backward(o),
    lambda o: pins.test_dense_equals_twell_sparse_bitwise(o, "int"),
    lambda o: pins.test_twell_roundtrip_and_counts(o),
    lambda o: pins.test_twell_width_cap(o),
    lambda o: pins.test_hybrid_invariants(o),
    lambda o: pins.test_forward_matches_torch(o),
    lambda o: pins.test_backward_matches_autograd(o, 5, 0.0),
    lambda o: pins.test_backward_matches_autograd(o, 5, 0.375),
    lambda o: pins.test_brute_force_tiny_layer(o),
    lambda o: pins.test_hybrid_forward_equals_twell_forward(o, "int"),
    lambda o: pins.test_hybrid_forward_matches_torch(o),
]


def _pins_fail(o) -> bool:
    for f in PIN_FUNCS:
        try:
            f(o)
        except AssertionError:
            return True
    return False


@pytest.fixture(scope="module")
def restore():
    yield
    orc_mod.load(orc_mod.LIB)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, restore):
    src = open(orc_mod.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site not unique: {name}"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mut.c")
        so = os.path.join(d, "libmut.so")
        open(c, "w").write(src.replace(old, new))
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-o", so, c])
        orc_mod.load(so)
        try:
            assert _pins_fail(orc_mod), f"no pin caught mutant: {name}"
        finally:
            orc_mod.load(orc_mod.LIB)


def test_unmutated_oracle_passes_pins(restore):
    orc_mod.load(orc_mod.LIB)
    assert not _pins_fail(orc_mod)
