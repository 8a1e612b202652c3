"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant is a copy of oracle/q4_oracle.c with one plausible mistake
planted in it (a swapped nibble order, a wrong signed offset, a wrong group
index, a dropped bias, a reversed contraction, ties rounded away from zero,
...).  The copy is compiled with the same flags into a temporary library, the
oracle module is pointed at it, and the pins of tests/test_oracle.py and
tests/test_oracle_next.py are run: every mutant must make at least one pin
fail.  Every planted mistake keeps all memory accesses in bounds.
"""
import os
import subprocess

import pytest

from oracle import build as obuild
from oracle import q4_oracle as orc
from tests import test_oracle as T1
from tests import test_oracle_next as T2

SRC = os.path.join(os.path.dirname(obuild.__file__), "q4_oracle.c")

# (name, text in q4_oracle.c, replacement); each text occurs exactly once
MUTANTS = [
    ("nibble order swapped", "return k_is_even ? low : high;", "return k_is_even ? high : low;"),
    ("signed offset 7", "return raw_code(qw, ldq, n, k, order) - 8;",
     "return raw_code(qw, ldq, n, k, order) - 7;"),
    ("first k of a group in group 0", "return scales[(k / gs) * lds + n];",
     "return scales[(k % gs == 0 ? 0 : k / gs) * lds + n];"),
    ("bias dropped", "acc += (double)bias[n];", "acc += 0.0;"),
    ("weight sign flipped", "    return (double)signed_code(qw, ldq, n, k, order) *",
     "    return -(double)signed_code(qw, ldq, n, k, order) *"),
    ("normaliser without abs", "        d += fabs(p);\n    }\n    if (bias)",
     "        d += p;\n    }\n    if (bias)"),
    ("binary16 ties away from zero", "double f = rint(a / quantum);  /* in [1024, 2048] */",
     "double f = floor(a / quantum + 0.5);  /* in [1024, 2048] */"),
    ("gradient contraction reversed", "double p = (double)dout[m * lddo + n] * wcol[n];",
     "double p = (double)dout[m * lddo + n] * wcol[N - 1 - n];"),
    ("requant ties away from zero", "float r = nearbyintf(q);", "float r = roundf(q);"),
    ("requant zero scale gives 0", "    if (s == 0.0f)\n        return 8;",
     "    if (s == 0.0f)\n        return 0;"),
    ("requant odd-K pad 0", "                            : 8;", "                            : 0;"),
    ("requant order swapped", "qw[n * ldq + b] = order == 0 ?", "qw[n * ldq + b] = order != 0 ?"),
    ("binary16 scale sign dropped", "dst[i] = (float)q4o_f16_value(h[i]);",
     "dst[i] = (float)q4o_f16_value(h[i] & 0x7FFF);"),
    ("binary16 subnormal read as normal", "v = ldexp((double)f, -24);",
     "v = ldexp((double)(1024 + f), -25);"),
]

PINS = [
    (T1.test_golden_worked_examples, {}),
    (T1.test_p1_every_byte_both_orders, dict(order="low_first")),
    (T1.test_p1_every_byte_both_orders, dict(order="high_first")),
    (T1.test_p2_all_eights_give_bias, dict(K=33, gs=8)),
    (T1.test_p3_scale_indexing, dict(K=12, N=5, gs=4, lds=7, order="low_first")),
    (T1.test_p4_exact_integer_case, dict(M=3, K=64, N=17, gs=32)),
    (T1.test_p5_linear_in_scale, {}),
    (T1.test_p7_dense_matmul, dict(M=7, K=300, N=50, gs=32, order="low_first")),
    (T1.test_p8_metamorphic, {}),
    (T1.test_rn_f16_matches_torch_conversion, {}),
    (T2.test_backward_dense_matmul, dict(M=5, K=300, N=70, gs=32, order="low_first")),
    (T2.test_backward_adjoint_of_forward, {}),
    (T2.test_requant_round_trip, dict(K=7, gs=3, order="high_first")),
    (T2.test_requant_ties_to_even_and_clamp, {}),
    (T2.test_requant_zero_scale_and_nan, {}),
    (T2.test_requant_packing_against_test_packer, {}),
    (T2.test_requant_golden, {}),
    (T2.test_f16_scale_values_every_pattern, {}),
    (T2.test_f16_scales_worked_example, {}),
]


def _pins_fail():
    failed = []
    for fn, kw in PINS:
        try:
            fn(**kw)
        except AssertionError:
            failed.append(fn.__name__)
    return failed


@pytest.fixture
def oracle_swap(monkeypatch, tmp_path):
    def use(src_text, tag):
        c = tmp_path / f"m_{tag}.c"
        so = tmp_path / f"m_{tag}.so"
        c.write_text(src_text)
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
                        "-fno-fast-math", "-shared", "-fPIC", str(c), "-o", str(so), "-lm"],
                       check=True, capture_output=True)
        monkeypatch.setattr(obuild, "LIB", str(so))
        monkeypatch.setattr(orc, "_lib", None)
    yield use
    monkeypatch.setattr(orc, "_lib", None)


def test_unmutated_copy_passes_every_pin(oracle_swap):
    oracle_swap(open(SRC).read(), "none")
    assert _pins_fail() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_mutant_fails_a_pin(oracle_swap, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    oracle_swap(src.replace(old, new), str(abs(hash(name))))
    failed = _pins_fail()
    assert failed, f"no pin caught the planted mistake: {name}"
