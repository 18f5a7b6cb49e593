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


# slips in the backward pass (oracle_bwd), each caught by its pins
BWD_MUTANTS = {
    "bwd_dk_term_dropped": ("a += G[(size_t)r * dv + c] * e[c] - St[(size_t)r * dv + c] * u[c];",
                            "a += G[(size_t)r * dv + c] * e[c];"),
    "bwd_dbeta_uses_v": ("db += u[c] * e[c];", "db += u[c] * (double)vt[c];"),
    "bwd_gate_grad_after_token": ("const double* S0i = Sb + (size_t)(i * nh) * SS;",
                                  "const double* S0i = So + (size_t)i * SS;"),
    "bwd_erase_not_propagated": ("G[(size_t)r * dv + c] -= bt * (double)kt[r] * u[c];",
                                 "G[(size_t)r * dv + c] -= 0.0 * bt * (double)kt[r] * u[c];"),
    "bwd_dq_unscaled": ("dqi[r] = scale * a;", "dqi[r] = a;"),
    "bwd_gate_not_applied": ("for (size_t x = 0; x < SS; ++x) G[x] *= g;", ""),
}

BWD_PINS = [
    lambda: P.test_bwd_matches_finite_differences(2, True, True),
    lambda: P.test_bwd_matches_finite_differences(1, False, False),
    P.test_bwd_one_token_closed_form,
]


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_planted_backward_mistake_is_caught(name, tmp_path, monkeypatch):
    a, b = BWD_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(a) == 1, name
    (tmp_path / "m.c").write_text(src.replace(a, b))
    so = tmp_path / "libm.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(tmp_path / "m.c"),
                    "-lm"], check=True)
    oracle._load()
    import ctypes
    lib = ctypes.CDLL(str(so))
    for f in ("oracle_fwd", "oracle_bwd"):
        getattr(lib, f).argtypes = getattr(oracle._lib, f).argtypes
        getattr(lib, f).restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for pin in BWD_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, name


# slips in the KDA recurrence (oracle_fwd_kda), each caught by its pins
KDA_MUTANTS = {
    "kda_decay_on_columns": ("const double a = exp((double)a_log[row * dk + r]);\n                for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= a;",
                             "for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= exp((double)a_log[row * dk + c % dk]);"),
    "kda_decay_twice": ("            const float* qi = q + row * dk;\n            double* oi = O + row * dv;",
                              "            for (int r = 0; r < dk; ++r) for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= exp((double)a_log[row * dk + r]) / exp((double)a_log[row * dk + r]) * exp((double)a_log[row * dk + r]);\n            const float* qi = q + row * dk;\n            double* oi = O + row * dv;"),
}

KDA_PINS = [P.test_kda_dplr_reduction, P.test_kda_equal_channels_is_gated_deltanet,
            P.test_kda_zero_channel_decay_erases_row]


@pytest.mark.parametrize("name", sorted(KDA_MUTANTS))
def test_planted_kda_mistake_is_caught(name, tmp_path, monkeypatch):
    a, b = KDA_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(a) == 1, name
    (tmp_path / "m.c").write_text(src.replace(a, b))
    so = tmp_path / "libm.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(tmp_path / "m.c"),
                    "-lm"], check=True)
    oracle._load()
    import ctypes
    lib = ctypes.CDLL(str(so))
    for f in ("oracle_fwd", "oracle_fwd_kda"):
        getattr(lib, f).argtypes = getattr(oracle._lib, f).argtypes
        getattr(lib, f).restype = ctypes.c_int
    monkeypatch.setattr(oracle, "_lib", lib)
    caught = 0
    for pin in KDA_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, name


# ---- the layer prologue/epilogue oracle (numpy): slips planted by swapping in a wrong function

def _conv_taps_reversed(x, w):
    return _REAL_CONV(x, w[:, ::-1])


def _l2_over_heads(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-2, keepdims=True) + eps)


def _silu_sigmoid_only(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def _epilogue_sum_not_mean(o, g, weight, eps=1e-6):
    o = np.asarray(o, dtype=np.float64)
    return o / np.sqrt(np.sum(o * o, axis=-1, keepdims=True) + eps) * weight * _REAL_SILU(g)


import numpy as np  # noqa: E402
from oracle import layer as _L  # noqa: E402
import test_oracle_layer as LP  # noqa: E402

_REAL_CONV, _REAL_SILU = _L.short_conv, _L.silu
LAYER_MUTANTS = {"conv_taps_reversed": ("short_conv", _conv_taps_reversed),
                 "l2_over_heads": ("l2_norm", _l2_over_heads),
                 "silu_is_sigmoid": ("silu", _silu_sigmoid_only),
                 "rms_sum_not_mean": ("epilogue", _epilogue_sum_not_mean)}
LAYER_PINS = [LP.test_silu_closed_forms, lambda: LP.test_conv_matches_numpy_convolve(4),
              LP.test_conv_current_tap_is_identity_and_causal, LP.test_prologue_unit_norm_and_direction,
              LP.test_epilogue_rms_gate_and_scale_invariance]


@pytest.mark.parametrize("name", sorted(LAYER_MUTANTS))
def test_planted_layer_mistake_is_caught(name, monkeypatch):
    attr, fn = LAYER_MUTANTS[name]
    monkeypatch.setattr(_L, attr, fn)
    failed = 0
    for pin in LAYER_PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, name
