"""Planted mistakes: every plausible slip in the oracle must fail at least one pin.

Each case copies the oracle's source, applies one textual mutation (a flipped
sign, a dropped term, a swapped operand), builds or loads the copy in a
temporary directory, and runs the pins of ``test_oracle_pins`` against it.
The committed oracle itself is never modified.
"""
import ctypes
import importlib.util
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_DIR = os.path.join(os.path.dirname(HERE), "oracle")

C_MUTATIONS = {
    "delta_sign": ("d[j] = bt * (vt[j] - acc);", "d[j] = bt * (vt[j] + acc);"),
    "no_decay": ("S[(int64_t)i * V + j] *= a;", "S[(int64_t)i * V + j] *= 1.0;"),
    "exp_not_exp2": ("g_is_log2 ? exp2(gt[i]) : exp(gt[i])", "exp(gt[i])"),
    "key_for_query": ("acc += S[(int64_t)i * V + j] * qt[i];", "acc += S[(int64_t)i * V + j] * kt[i];"),
    "no_scale": ("ot[j] = acc * scale;", "ot[j] = acc;"),
    "no_beta": ("d[j] = bt * (vt[j] - acc);", "d[j] = (vt[j] - acc);"),
    "sigmoid_sign": ("(1.0 / (1.0 + exp(-a)))", "(1.0 / (1.0 + exp(a)))"),
    "softplus_log": ("? z : log1p(exp(z))", "? z : log(exp(z) + 0.5)"),
    "no_dt_bias": ("x[idx] + (dt_bias ? dt_bias[(int64_t)h * K + i] : 0.0)", "x[idx]"),
    "transposed_state_read": ("acc += S[(int64_t)i * V + j] * kt[i];",
                              "acc += S[(int64_t)(j % K) * V + (i % V)] * kt[i];"),
}

# slips in the reverse-mode pass; each must fail the finite-difference pin
BWD_MUTATIONS = {
    "bwd_dq_no_scale": ("dqt[i] = scale * acc;", "dqt[i] = acc;"),
    "bwd_dk_sign": ("dkt[i] = a1 - bt * a2;", "dkt[i] = a1 + bt * a2;"),
    "bwd_dg_no_alpha": ("dgt[i] = al * acc;", "dgt[i] = acc;"),
    "bwd_no_decay_carry": ("dS[(int64_t)i * V + j] = al * dp;", "dS[(int64_t)i * V + j] = dp;"),
    "bwd_dbeta_drops_state": ("db += acc * (vt[j] - u[j]);", "db += acc * vt[j];"),
    "bwd_dp_without_beta": ("double dp = dS[(int64_t)i * V + j] - bt * kt[i] * ddl[j];",
                            "double dp = dS[(int64_t)i * V + j] - kt[i] * ddl[j];"),
    "bwd_dg_against_new_state": ("acc += dp * Sp[(int64_t)i * V + j];", "acc += dp * St[(int64_t)i * V + j];"),
}

PY_MUTATIONS = {
    "diag_in_Akk": ("Akk = np.tril(Akk, -1) * bc[:, None]", "Akk = np.tril(Akk) * bc[:, None]"),
    "no_state_decay": ("h_next = np.exp2(bL)[:, None] * h +", "h_next = h +"),
    "vnew_sign": ("vnew = u - w @ h", "vnew = u + w @ h"),
    "w_without_gamma": ("w = Tm @ (bc[:, None] * kc * gam)", "w = Tm @ (bc[:, None] * kc)"),
    "q_without_gamma": ("o = scale * (qc * gam) @ h", "o = scale * qc @ h"),
    "beta_in_columns": ("Akk = np.tril(Akk, -1) * bc[:, None]", "Akk = np.tril(Akk, -1) * bc[None, :]"),
    "offdiag_anchor_wrong_side": ("col = np.exp2(a - b[S])", "col = np.exp2(b[S] - a)"),
    "k_tilde_direction": ("(kc * np.exp2(bL - b)).T @ vnew", "(kc * np.exp2(b - bL)).T @ vnew"),
}

CUMSUM_MUTATIONS = {
    "no_chunk_restart": ("            if (t - s0) % C == 0:\n", "            if t == s0:\n"),
    "restart_on_absolute_row": ("            if (t - s0) % C == 0:\n", "            if t % C == 0:\n"),
    "exclusive_cumsum": ("            run = run + gf[t] * unit\n            out[t] = run\n",
                         "            out[t] = run\n            run = run + gf[t] * unit\n"),
    "natural_log_units": ("unit = 1.0 if g_is_log2 else RCP_LN2", "unit = 1.0"),
}

RECURRENCE_PINS = [
    ("test_exact_bruteforce_dyadic", dict(K=4, V=4, T=6, seed=0)),
    ("test_scalar_closed_form", {}),
    ("test_zero_gate_is_plain_delta_rule", {}),
    ("test_zero_beta_pure_decay", {}),
    ("test_small_beta_limit_is_gated_linear_attention", {}),
    ("test_unit_beta_query_equals_key", {}),
    ("test_axis_aligned_keys_decouple_rows", {}),
    ("test_gate_activations", {}),
]

CHUNKED_PINS = [
    ("test_chunked_matches_recurrence", dict(C=64, anchored=True, mid=8, gate="safe")),
    ("test_chunked_matches_recurrence", dict(C=32, anchored=False, mid=8, gate="softplus")),
    ("test_chunked_packed_and_intermediates", {}),
    ("test_chunked_gram_matches_pairwise_definition", {}),
]


def _fails_some_pin(pin_list):
    for name, kw in pin_list:
        try:
            getattr(pins, name)(oracle, **kw)
        except (AssertionError, FloatingPointError, ValueError, np_linalg_error()):
            return True
    return False


def np_linalg_error():
    import numpy as np

    return np.linalg.LinAlgError


@pytest.mark.parametrize("name", sorted(C_MUTATIONS))
def test_c_mutation_is_caught(oracle_mod, tmp_path, name):
    src = open(os.path.join(ORACLE_DIR, "kda_oracle.c")).read()
    old, new = C_MUTATIONS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous: " + old
    mutated = tmp_path / "m.c"
    mutated.write_text(src.replace(old, new, 1))
    so = tmp_path / "libm.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutated), "-o", str(so), "-lm"],
                   check=True)
    good = oracle._lib()
    lib = ctypes.CDLL(str(so))
    lib.kda_oracle_gate.argtypes = good.kda_oracle_gate.argtypes
    lib.kda_oracle_recurrent.argtypes = good.kda_oracle_recurrent.argtypes
    saved = oracle._LIB
    oracle._LIB = lib
    try:
        assert _fails_some_pin(RECURRENCE_PINS), "mutation %s survived every pin" % name
    finally:
        oracle._LIB = saved


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_bwd_mutation_is_caught(oracle_mod, tmp_path, name):
    src = open(os.path.join(ORACLE_DIR, "kda_oracle.c")).read()
    old, new = BWD_MUTATIONS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous: " + old
    mutated = tmp_path / "m.c"
    mutated.write_text(src.replace(old, new, 1))
    so = tmp_path / "libm.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutated), "-o", str(so), "-lm"],
                   check=True)
    good = oracle._lib()
    lib = ctypes.CDLL(str(so))
    for fn in ("kda_oracle_gate", "kda_oracle_recurrent", "kda_oracle_recurrent_bwd"):
        getattr(lib, fn).argtypes = getattr(good, fn).argtypes
    saved = oracle._LIB
    oracle._LIB = lib
    try:
        assert _fails_some_pin([("test_recurrent_bwd_finite_differences", {})]), \
            "mutation %s survived every pin" % name
    finally:
        oracle._LIB = saved


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_chunked_mutation_is_caught(oracle_mod, tmp_path, name):
    src = open(os.path.join(ORACLE_DIR, "chunked.py")).read()
    old, new = PY_MUTATIONS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous: " + old
    path = tmp_path / "chunked_mut.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("chunked_mut_%s" % name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    saved = pins.chunked_forward
    pins.chunked_forward = mod.chunked_forward
    try:
        assert _fails_some_pin(CHUNKED_PINS), "mutation %s survived every pin" % name
    finally:
        pins.chunked_forward = saved


@pytest.mark.parametrize("name", sorted(CUMSUM_MUTATIONS))
def test_cumsum_mutation_is_caught(oracle_mod, tmp_path, name):
    src = open(os.path.join(ORACLE_DIR, "chunked.py")).read()
    old, new = CUMSUM_MUTATIONS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous: " + old
    path = tmp_path / "cumsum_mut.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("cumsum_mut_%s" % name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    saved = pins.chunk_cumsum_log2
    pins.chunk_cumsum_log2 = mod.chunk_cumsum_log2
    try:
        assert _fails_some_pin([("test_chunk_cumsum_pins", {})]), "mutation %s survived every pin" % name
    finally:
        pins.chunk_cumsum_log2 = saved


L2NORM_MUTATIONS = {
    "no_eps": ("keepdims=True) + eps)", "keepdims=True))"),
    "wrong_axis": ("axis=-1", "axis=0"),
    "no_sqrt": ("np.sqrt(np.sum", "(np.sum"),
    "no_square": ("np.sum(x * x,", "np.sum(np.abs(x),"),
}


@pytest.mark.parametrize("name", sorted(L2NORM_MUTATIONS))
def test_l2norm_mutation_is_caught(name):
    import inspect
    import types

    import numpy as np

    src = inspect.getsource(oracle.l2norm_rows)
    old, new = L2NORM_MUTATIONS[name]
    assert src.count(old) == 1, "mutation anchor missing or ambiguous: " + old
    ns = {"np": np, "L2NORM_EPS": oracle.L2NORM_EPS, "_f64": oracle._f64}
    exec(src.replace(old, new, 1), ns)
    fake = types.SimpleNamespace(l2norm_rows=ns["l2norm_rows"])
    with pytest.raises(AssertionError):
        pins.test_l2norm_rows_pins(fake)

