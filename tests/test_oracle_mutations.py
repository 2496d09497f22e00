"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of oracle/osdn_oracle.c (on the
CPU, never in the committed source), builds it, swaps it in for the real
oracle, and runs the pin tests: at least one of them has to fail.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "osdn_oracle.c")

EMIT = "for (int64_t i = 0; i < K; ++i) out[i] = d[i] * kt[i];"
MUTATIONS = {
    "write_key_not_scaled": [("out[i] = d[i] * kt[i]", "out[i] = kt[i]")],
    "emit_after_update": [(EMIT, ""), ("d[i] = x;", "d[i] = x; out[i] = d[i] * kt[i];")],
    "step_sign_flipped": [("double c = eta * bp", "double c = -eta * bp")],
    "beta_dropped_in_alignment": [("(1.0 - bp * align)", "(1.0 - align)")],
    "no_key_norm": [("(1.0 - bp * align) / n;", "(1.0 - bp * align);")],
    "retention_on_step_too": [("rt * d[i] + c * s[i]", "rt * (d[i] + c * s[i])")],
    "no_clamp": [("if (clamp) {", "if (0) {")],
    "read_with_write_key": [("acc += S[i * K + j] * kt[j];\n        u[i]",
                             "acc += S[i * K + j] * wt[j];\n        u[i]")],
    "write_with_read_key": [("bt * u[i] * wt[j]", "bt * u[i] * kt[j]")],
    "write_gate_dropped": [("bt * u[i] * wt[j]", "u[i] * wt[j]")],
    "q_scale_ignored": [("(q_scale * qt[j])", "qt[j]")],
    "decay_ignored": [("S[e] *= at;", "S[e] *= 1.0;")],
    "decay_applied_after_read": [
        ("for (size_t e = 0; e < VK; ++e) S[e] *= at;\n      }", "}"),
        ("if (u_out)", "if (alpha) { double at = alpha[at_bth(b, t, h, T, H)];"
                       " for (size_t e = 0; e < VK; ++e) S[e] *= at; }\n      if (u_out)")],
}


def _pin_tests(module=pins):
    out = []
    for name in dir(module):
        fn = getattr(module, name)
        if name.startswith("test_") and callable(fn):
            marks = getattr(fn, "pytestmark", [])
            params = [m for m in marks if m.name == "parametrize"]
            if not params:
                out.append((name, fn, {}))
                continue
            combos = [{}]
            for m in params:
                argnames = [a.strip() for a in m.args[0].split(",")]
                new = []
                for c in combos:
                    for val in m.args[1]:
                        vals = val if len(argnames) > 1 else (val,)
                        d = dict(c)
                        d.update(zip(argnames, vals))
                        new.append(d)
                combos = new
            out.extend((name, fn, c) for c in combos)
    return out


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_mutation(mutation, tmp_path, monkeypatch):
    src = open(SRC).read()
    for old, new in MUTATIONS[mutation]:
        assert old in src, "mutation anchor missing: %r" % old
        src = src.replace(old, new, 1)
    cfile = tmp_path / "mut.c"
    cfile.write_text(src)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                    str(so), str(cfile), "-lm"], check=True)
    lib = oracle.bind(ctypes.CDLL(str(so)))
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for name, fn, kwargs in _pin_tests():
        try:
            fn(oracle_lib=oracle, **kwargs) if "oracle_lib" in fn.__code__.co_varnames else fn(**kwargs)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    assert failed, "no pin caught the planted mistake %s" % mutation


# ---- OSKDA phase 2 and vector retention: the pins of tests/test_oracle_kda.py
KDA_MUTATIONS = {
    "kda_decay_ignored": [("S[i * V + j] *= at[i];", "S[i * V + j] *= 1.0;")],
    "kda_decay_on_value_axis": [("S[i * V + j] *= at[i];", "S[i * V + j] *= at[j % K];")],
    "kda_read_with_write_key": [("acc += S[i * V + j] * kt[i];", "acc += S[i * V + j] * wt[i];")],
    "kda_write_with_read_key": [("bt * wt[i] * u[j]", "bt * kt[i] * u[j]")],
    "kda_write_gate_dropped": [("bt * wt[i] * u[j]", "wt[i] * u[j]")],
    "kda_readout_from_old_state": [
        ("for (int64_t i = 0; i < K; ++i)\n        for (int64_t j = 0; j < V; ++j) S[i * V + j] += bt * wt[i] * u[j];\n", ""),
        ("    for (size_t e = 0; e < KV; ++e) S_out[(size_t)bh * KV + e] = S[e];",
         "    for (size_t e = 0; e < KV; ++e) S_out[(size_t)bh * KV + e] = S[e] + 0.0 * u[0];")],
    "kda_q_scale_ignored": [("(q_scale * qt[i]);\n        ot[j] = acc;", "qt[i];\n        ot[j] = acc;")],
    "vector_retention_first_entry_only": [("r[at_bthx(b, t, h, i, T, H, K)]", "r[at_bthx(b, t, h, 0, T, H, K)]")],
    "vector_retention_ignored": [("r_per_key ? r[at_bthx(b, t, h, i, T, H, K)]", "r_per_key ? 1.0")],
}


@pytest.mark.parametrize("mutation", sorted(KDA_MUTATIONS))
def test_kda_pins_catch_mutation(mutation, tmp_path, monkeypatch):
    from tests import test_oracle_kda as kpins
    src = open(SRC).read()
    for old, new in KDA_MUTATIONS[mutation]:
        assert old in src, "mutation anchor missing: %r" % old
        src = src.replace(old, new, 1)
    cfile = tmp_path / "mut.c"
    cfile.write_text(src)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                    str(so), str(cfile), "-lm"], check=True)
    lib = oracle.bind(ctypes.CDLL(str(so)))
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for name, fn, kwargs in _pin_tests(kpins):
        try:
            fn(**kwargs)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    assert failed, "no pin caught the planted mistake %s" % mutation


# ---- backward oracle: each planted mistake must fail a finite-difference pin
BWD_SRC = os.path.join(os.path.dirname(oracle.__file__), "osdn_oracle_bwd.c")
BWD_MUTATIONS = {
    "readout_gradient_missing": [("G[i * K + jj] += q_scale * dot[i] * qt[jj];", "")],
    "dq_unscaled": [("dqt[jj] = q_scale * acc;", "dqt[jj] = acc;")],
    "dv_without_gate": [("dvt[i] = bt * acc;", "dvt[i] = acc;")],
    "write_key_gradient_from_w": [("acc += G[i * K + jj] * uj[i];", "acc += G[i * K + jj] * w[i];")],
    "read_key_gradient_sign": [("dkt_read[jj] = -bt * acc;", "dkt_read[jj] = bt * acc;")],
    "residual_term_dropped": [("dSb[i * K + jj] = G[i * K + jj] - bt * w[i] * kt[jj];",
                               "dSb[i * K + jj] = G[i * K + jj];")],
    "decay_not_propagated": [("G[e] = at * dSb[e];", "G[e] = dSb[e];")],
    "decay_gradient_wrong_state": [("da += dSb[e] * Sp[e];", "da += dSb[e] * St[e];")],
    "clamp_mask_ignored": [("gy[i] = pass ? g[i] : 0.0;", "gy[i] = g[i];")],
    "norm_floor_ignored": [("nraw > eps ? -c / n : 0.0", "-c / n")],
    "write_key_path_to_k_missing": [(" + dktil[i] * d[i];", ";")],
    "retention_not_in_carry": [("+ rt * gy[i] +", "+ gy[i] +")],
    "beta_aware_step_term_missing": [
        ("if (beta_aware) dbeta[bw_bth(b, t, h, T, H)] += gc * eta * (1.0 - 2.0 * bp * a) / n;", "")],
    "alignment_term_missing": [("+ gc * dca * d[i] +", " +")],
}


@pytest.mark.parametrize("mutation", sorted(BWD_MUTATIONS))
def test_backward_pins_catch_mutation(mutation, tmp_path, monkeypatch):
    from tests import test_oracle_backward as bpins
    src = open(BWD_SRC).read()
    for old, new in BWD_MUTATIONS[mutation]:
        assert old in src, "mutation anchor missing: %r" % old
        src = src.replace(old, new, 1)
    cfile = tmp_path / "mut_bwd.c"
    cfile.write_text(src)
    so = tmp_path / "libmutbwd.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o",
                    str(so), SRC, str(cfile), "-lm"], check=True)
    lib = oracle.bind(ctypes.CDLL(str(so)))
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for name in bpins.CASES:
        try:
            bpins.test_backward_matches_finite_differences(name)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    assert failed, "no backward pin caught the planted mistake %s" % mutation
