"""The pins are strong enough: plausible mistakes planted in a copy of the oracle fail them.

Each mutant is the oracle's C source with one textual change (a dropped term, a wrong sign,
a gate on the wrong axis, a wrong operand or index), built with gcc into a temporary library.
The planted mistakes live only in these temporary copies, on the CPU.
"""
import os
import shutil

import pytest

import oracle
import oracle_pins as P

MUTANTS = {
    "decay_dropped": ("S[i * dv + c] *= a[i];", "S[i * dv + c] *= 1.0;"),
    "decay_on_value_axis": ("S[i * dv + c] *= a[i];", "S[i * dv + c] *= a[c % dk];"),
    "erase_sign_flipped": ("S[i * dv + c] -= k[i] * r[c];", "S[i * dv + c] += k[i] * r[c];"),
    "erase_term_dropped": ("S[i * dv + c] -= k[i] * r[c];", "S[i * dv + c] -= 0.0 * r[c];"),
    "erase_gate_dropped": ("const double e = be[i] * k[i];", "const double e = k[i];"),
    "erase_reads_query": ("const double e = be[i] * k[i];", "const double e = be[i] * q[i];"),
    "write_gate_dropped": ("k[i] * (w[c] * v[c])", "k[i] * (v[c])"),
    "write_gate_on_key_axis": ("k[i] * (w[c] * v[c])", "k[i] * (be[i] * v[c])"),
    "readout_with_key": ("o[c] += q[i] * S[i * dv + c];", "o[c] += k[i] * S[i * dv + c];"),
    "readout_transposed": ("o[c] += q[i] * S[i * dv + c];",
                           "o[c] += q[i] * S[(c % dk) * dv + (i % dv)];"),
    "initial_state_ignored": ("if (j->S0) {", "if (0) {"),
    "head_index_dropped": ("const long tok = (bb * j->T + t) * j->H + hh;",
                           "const long tok = (bb * j->T + t) * j->H;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(oracle._SRC).read()
    # the forward pass is everything before the backward's section (which recomputes states
    # with the same lines; its own mutants live in tests/test_oracle_bwd.py)
    cut = src.index("/*\n * Backward:")
    fwd_src, rest = src[:cut], src[cut:]
    assert fwd_src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = os.path.join(mutant_dir, name + ".c")
    with open(path, "w") as f:
        f.write(fwd_src.replace(old, new) + rest)
    lib = oracle.load_library(oracle.build(force=True, out_path=path[:-2] + ".so", src_path=path))

    def fwd(q, k, v, alpha, b, w, S0):
        return oracle.forward(q, k, v, alpha, b, w, S0, threads=1, lib=lib)

    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(fwd)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
