"""The oracle's pins are sensitive: plausible slips planted in a copy of oracle.c (on the CPU,
never in the GPU path) each make at least one pin fail."""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "residual_sign": ("e[c] -= Sr[c] * kr;", "e[c] += Sr[c] * kr;"),
    "beta_dropped": ("const double a = bt * (double)kt[r];", "const double a = (double)kt[r];"),
    "substeps_reversed": ("const long t = i * nh + j;", "const long t = i * nh + (nh - 1 - j);"),
    "gate_twice": ("S[x] *= g;", "S[x] *= g * g;"),
    "readout_transposed": ("oi[c] += Sr[c] * qr;", "oi[c] += S[(size_t)c * dv + r] * qi[c % dk];"),
}

PINS = [
    lambda: P.test_householder_eigenvalues(0.3),
    lambda: P.test_exact_write_beta_one(True),
    P.test_mod3_rotation_golden,
    P.test_nh2_cross_term,
    lambda: P.test_brute_force_products(2, True, True),
    lambda: P.test_chunked_form_matches(8, 1, True),
    P.test_dplr_reductions,
    P.test_one_chunk_closed_form,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    a, b = MUTANTS[name]
    src = open(SRC).read()
    assert a in src
    (tmp_path / "m.c").write_text(src.replace(a, b))
    so = tmp_path / "libm.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(tmp_path / "m.c"),
                    "-lm"], check=True)
    oracle._load()                       # make sure the real library's argtypes are set up
    import ctypes
    lib = ctypes.CDLL(str(so))
    lib.oracle_fwd.argtypes = oracle._lib.oracle_fwd.argtypes
    lib.oracle_fwd.restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, name
