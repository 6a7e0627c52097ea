"""The CPU oracle against the pages' printed values, closed forms and invariants,
plus mutation checks showing that plausible mistakes in the oracle fail a pin."""
import importlib.util
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build

from . import oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(lib, pin):
    pin(lib)


def test_checked_step_matches_worked_example():
    # tests/golden/worked_example.json: the tutorial's two-cell example and its two printed results
    for case in pins.golden()["cases"]:
        got = oracle.checked_step(case["state"], case["key"], case["value"], case["alpha"], case["beta"])
        assert np.array_equal(got, np.array(case["expected"]))


@pytest.mark.parametrize("args", [
    ([], [1.0], [1.0], 0.5, 0.5),                      # empty state
    ([[1.0, 2.0]], [], [1.0], 0.5, 0.5),               # empty key
    ([[1.0, 2.0]], [1.0, 0.0], [1.0, 2.0], 0.5, 0.5),  # value/state rows mismatch
    ([[1.0, 2.0, 3.0]], [1.0, 0.0], [1.0], 0.5, 0.5),  # row length != key length
    ([1.0, 2.0], [1.0, 0.0], [1.0], 0.5, 0.5),         # state not a matrix
    ([[float("nan"), 2.0]], [1.0, 0.0], [1.0], 0.5, 0.5),
    ([[1.0, 2.0]], [1.0, 0.0], [float("inf")], 0.5, 0.5),
    ([[1.0, 2.0]], [1.0, 0.0], [1.0], float("nan"), 0.5),
    ([[1.0, 2.0]], [1.0, 0.0], [1.0], 1.5, 0.5),       # decay outside [0, 1]
    ([[1.0, 2.0]], [1.0, 0.0], [1.0], 0.5, -0.1),      # write outside [0, 1]
    ([[1.0, 2.0]], [1.0, 1.0], [1.0], 0.5, 0.5),       # key not unit
])
def test_checked_step_rejects(args):
    with pytest.raises(ValueError):
        oracle.checked_step(*args)


def test_checked_step_endpoints():
    # alpha = 0 wipes the memory before the write; beta = 0 only decays.
    assert np.array_equal(oracle.checked_step([[2.0, 10.0]], [1.0, 0.0], [6.0], 0.0, 0.25), [[1.5, 0.0]])
    assert np.array_equal(oracle.checked_step([[2.0, 10.0]], [0.0, 1.0], [6.0], 0.5, 0.0), [[1.0, 5.0]])


def test_malformed_cu_rejected(lib):
    q = np.zeros((1, 4, 1, 2))
    with pytest.raises(ValueError):
        oracle.recurrent(q, q, q, np.zeros((1, 4, 1)), np.zeros((1, 4, 1)),
                         cu_seqlens=np.array([0, 3, 2, 4]), lib=lib)


def test_intermediates_exposed():
    rng = np.random.default_rng(3)
    L, dk, dv = 70, 8, 5
    q = rng.standard_normal((L, dk))
    k = rng.standard_normal((L, dk)) / 3
    v = rng.standard_normal((L, dv))
    la = rng.uniform(-0.1, -0.01, L)
    b = rng.uniform(0.2, 0.8, L)
    _, _, inter = oracle.chunked_single(q, k, v, la, b, chunk=32, keep=True)
    assert len(inter) == 3 and inter[-1]["T"].shape == (6, 6)
    for it in inter:
        c = it["T"].shape[0]
        # T inverts I + A, A strictly lower, Gamma lower with unit diagonal.
        assert np.allclose(it["T"] @ (np.eye(c) + it["A"]), np.eye(c), atol=1e-12)
        assert np.allclose(np.triu(it["A"]), 0) and np.allclose(np.diag(it["Gamma"]), 1)
        assert np.allclose(np.triu(it["Gamma"], 1), 0)


# -- mutation checks: each planted mistake must fail at least one pin ---------

C_MUTANTS = {
    "wrong_error_sign": ("err[i] = beta * (v[i] - pred);", "err[i] = beta * (v[i] + pred);"),
    "dropped_beta": ("err[i] = beta * (v[i] - pred);", "err[i] = (v[i] - pred);"),
    "dropped_gate": ("const double alpha = exp(log_alpha);",
                     "const double alpha = 1.0 + 0.0 * log_alpha;"),
    "undecayed_error": ("pred += S[i * dk + j] * k[j];", "pred += S[i * dk + j] / alpha * k[j];"),
    "predict_with_q": ("pred += S[i * dk + j] * k[j];", "pred += S[i * dk + j] * q[j];"),
    "write_along_q": ("S[i * dk + j] += err[i] * k[j];", "S[i * dk + j] += err[i] * q[j];"),
    "read_with_k": ("acc += S[i * dk + j] * q[j];\n        o[i] = acc;",
                    "acc += S[i * dk + j] * k[j];\n        o[i] = acc;"),
    "init_ignored": ("        if (init_state)\n            memcpy(S, init_state + (n * H + h) * dv * dk, sizeof(double) * (size_t)(dv * dk));\n        else",
                     "        if (0 && init_state)\n            memcpy(S, init_state + (n * H + h) * dv * dk, sizeof(double) * (size_t)(dv * dk));\n        else"),
    "beta_wrong_head": ("log_alpha[th], beta[th], o + th * dv);",
                        "log_alpha[th], beta[t * H], o + th * dv);"),
    "bwd_dq_from_previous_state": ("acc += Sc[i * dk + j] * dot[i];", "acc += Sp[i * dk + j] * dot[i];"),
    "bwd_dk_without_beta": ("acc += G[i * dk + j] * err[i] - b * alpha * Sp[i * dk + j] * de[i];",
                            "acc += G[i * dk + j] * err[i] - alpha * Sp[i * dk + j] * de[i];"),
    "bwd_dlog_alpha_not_scaled": ("dlog_alpha[th] = alpha * da;", "dlog_alpha[th] = da;"),
    "bwd_adjoint_not_decayed": ("G[i * dk + j] = alpha * dsb;", "G[i * dk + j] = dsb;"),
    "bwd_output_term_dropped": ("G[i * dk + j] += dot[i] * qt[j];", "G[i * dk + j] += 0.0 * dot[i] * qt[j];"),
}


def _fails_some_pin(lib, chunked_fn=None):
    failures = []
    for pin in pins.ALL_PINS:
        try:
            if pin is pins.pin_chunked_matches_recurrent and chunked_fn is not None:
                pin(lib, chunked_fn)
            else:
                pin(lib)
        except AssertionError:
            failures.append(pin.__name__)
    return failures


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(name, tmp_path):
    src = open(oracle_build.SRC).read()
    old, new = C_MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} no longer in the oracle source"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new, 1))
    so = oracle_build.build(str(tmp_path / "libmut.so"), str(mut))
    lib = oracle.load(so)
    assert _fails_some_pin(lib), f"mutant {name} passed every pin"


PY_MUTANTS = {
    "causal_mask_output": ("P = (Q @ K.T) * Gamma", "P = (Q @ K.T) * incl"),
    "w_without_decay": ("W_dec = T @ (b[:, None] * gam[:, None] * K)", "W_dec = T @ (b[:, None] * K)"),
    "k_decayed_from_start": ("K_end = np.exp(g[-1] - g)[:, None] * K", "K_end = np.exp(g)[:, None] * K"),
    "exclusive_cumsum": ("g = np.cumsum(la)", "g = np.cumsum(la) - la"),
    "a_without_gamma": ("A = np.tril(b[:, None] * (Gamma * (K @ K.T)), -1)",
                        "A = np.tril(b[:, None] * (K @ K.T), -1)"),
    "q_not_decayed": ("O = gam[:, None] * (Q @ S.T) + P @ Vp", "O = (Q @ S.T) + P @ Vp"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_chunked_mutant_is_caught(name, tmp_path, lib):
    path = os.path.join(ROOT, "oracle", "chunked.py")
    src = open(path).read()
    old, new = PY_MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} no longer in chunked.py"
    mut = tmp_path / "chunked_mut.py"
    mut.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("chunked_mut", str(mut))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises(AssertionError):
        pins.pin_chunked_matches_recurrent(lib, mod.chunked)
