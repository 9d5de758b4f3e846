"""The oracle's backward against its pins, and planted mistakes in copies of it caught by them."""
import os
import shutil

import numpy as np
import pytest

import oracle
import oracle_bwd_pins as P


@pytest.mark.parametrize("pin", P.ALL_BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    fwd = lambda q, k, v, alpha, b, w, S0: oracle.forward(q, k, v, alpha, b, w, S0, threads=1)
    bwd = lambda *a: oracle.backward(*a, threads=1)
    pin(bwd, fwd)


def test_bwd_threads_and_null_cotangents():
    """Thread count does not change the result; NULL dO / dS_T / S0 mean zeros."""
    rng = np.random.default_rng(21)
    q, k, v, alpha, b, w, S0 = __import__("oracle_pins").random_inputs(rng, 2, 67, 3, 4, 5)
    dO = rng.standard_normal((2, 67, 3, 5))
    g1 = oracle.backward(q, k, v, alpha, b, w, S0, dO, None, threads=1)
    g4 = oracle.backward(q, k, v, alpha, b, w, S0, dO, np.zeros((2, 3, 4, 5)), threads=4)
    for n in g1:
        np.testing.assert_array_equal(g1[n], g4[n])
    g0 = oracle.backward(q, k, v, alpha, b, w, None, None, None, threads=2)
    for n in g0:
        assert not np.any(g0[n]), n


BWD_MUTANTS = {
    "readout_uses_old_state": ("acc += St[i * dv + c] * dO[c];", "acc += P[i * dv + c] * dO[c];"),
    "write_term_dropped": ("acc += G[i * dv + c] * (w[c] * v[c]);", "acc += 0.0 * G[i * dv + c];"),
    "erase_sign_flipped": ("dk_o[i] -= acc;", "dk_o[i] += acc;"),
    "erase_read_dropped": ("G[i * dv + c] += cvec[i] * dr[c];", "G[i * dv + c] += 0.0 * dr[c];"),
    "decay_not_applied": ("for (long c = 0; c < dv; ++c) G[i * dv + c] *= a[i];",
                          "for (long c = 0; c < dv; ++c) G[i * dv + c] *= 1.0;"),
    "dalpha_from_decayed_state": ("acc += P[i * dv + c] * G[i * dv + c];", "acc += X[i * dv + c] * G[i * dv + c];"),
    "db_gate_swapped": ("db[i] = k[i] * acc;", "db[i] = be[i] * acc;"),
    "dw_dv_swapped": ("dv_o[c] = w[c] * acc;", "dv_o[c] = v[c] * acc;"),
    "checkpoint_off_by_one": ("memcpy(seg, ck + m * n, sizeof(double) * (size_t)n);",
                              "memcpy(seg, ck + (m > 0 ? m - 1 : 0) * n, sizeof(double) * (size_t)n);"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("oracle_bwd_mutants")


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(name, mutant_dir):
    old, new = BWD_MUTANTS[name]
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = os.path.join(mutant_dir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load_library(oracle.build(force=True, out_path=path[:-2] + ".so", src_path=path))
    fwd = lambda q, k, v, alpha, b, w, S0: oracle.forward(q, k, v, alpha, b, w, S0, threads=1)
    bwd = lambda *a: oracle.backward(*a, threads=1, lib=lib)
    failed = []
    for pin in P.ALL_BWD_PINS:
        try:
            pin(bwd, fwd)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every backward pin"
