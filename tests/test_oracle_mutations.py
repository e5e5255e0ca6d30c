"""Planted mistakes in the oracle must each fail at least one pin.

Each case copies ``oracle/fix_oracle.c`` to a temporary directory, applies one
plausible slip by text substitution (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one in the gate product), compiles that copy,
and runs every pin against it.  The shipped oracle is never modified.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle as O
from pins import ALL_PINS

SRC = open(os.path.join(os.path.dirname(O.__file__), "fix_oracle.c")).read()

MUTATIONS = {
    # gate of token j included in its own decay (exclusive-vs-inclusive slip)
    "decay_off_by_one": [(
        "    for (int64_t d = 0; d < dv; ++d) x[d] += p * D[d] * vj[d];\n"
        "    for (int64_t d = 0; d < dv; ++d) D[d] *= aj[d];",
        "    for (int64_t d = 0; d < dv; ++d) D[d] *= aj[d];\n"
        "    for (int64_t d = 0; d < dv; ++d) x[d] += p * D[d] * vj[d];")],
    "eps_dropped": [("sqrt(ss / c->dv + c->eps)", "sqrt(ss / c->dv)")],
    "scale_dropped": [("sc[j] = c->scale * dot(", "sc[j] = dot(")],
    "row_max_wrong": [("if (sc[j] > m) m = sc[j];", "if (j == 0) m = sc[j];")],
    "gqa_head_map": [("kh = h / c->G", "kh = h % c->Hkv"), ("kh = h / c.G", "kh = h % c.Hkv")],
    "delta_projection_dropped": [("delta[d] = r * (delta[d] - x[d] * r * proj)", "delta[d] = r * delta[d]")],
    "delta_projection_sign": [("delta[d] = r * (delta[d] - x[d] * r * proj)",
                               "delta[d] = r * (delta[d] + x[d] * r * proj)")],
    "dq_scale_dropped": [("dq[ro * dk + e2] = scale * acc[e2]", "dq[ro * dk + e2] = acc[e2]")],
    "dv_missing_prob": [("adv[d] += P * D[d] * delta[d];", "adv[d] += D[d] * delta[d];")],
    "dk_transposed_operand": [("adk[e2] += dS * qi[e2];", "adk[e2] += dS * kj[e2];")],
    "dG_sign": [("dG -= v[ko * dv + d] * dv_out[ko * dv + d];", "dG += v[ko * dv + d] * dv_out[ko * dv + d];")],
    "dg_forward_scan": [("for (int64_t t = L - 1; t >= lo; --t) {", "for (int64_t t = lo; t < L; ++t) {")],
    "dg_missing_query_term": [("dG += DL[ro * dv + d] * X[ro * dv + d];", "dG += 0.0;")],
    "dw_missing_rstd": [("acc += dn * X[ro * dv + d] * R[ro];", "acc += dn * X[ro * dv + d];")],
    "dz_uses_x": [("if (dz) dz[ro * dv + d] = dOr[d] * nval;", "if (dz) dz[ro * dv + d] = dOr[d] * x[d];")],
    "gate_weight_in_norm": [("if (o_norm) val = val * r * (w ? w[d] : 1.0);", "if (o_norm) val = val * r;")],
    "window_off_by_one": [("return L - c->window;", "return L - c->window + 1;")],
    "dkv_loop_skips_diagonal": [("for (int64_t i = j; i < L; ++i) {", "for (int64_t i = j + 1; i < L; ++i) {")],
    # the exact-zero shortcut of the decay walks taken when any channel (not every one) is zero
    "vanishing_shortcut_any_channel": [("    if (D[d] != 0.0) return 0;\n  return 1;", "    if (D[d] == 0.0) return 1;\n  return 0;")],
    # gate logits: sigmoid sign slip, and the chain-rule factor dropped or with the wrong sign
    "logits_sigmoid_sign": [("1.0 / (1.0 + exp(-g[e]))", "1.0 / (1.0 + exp(g[e]))")],
    "logits_chain_rule_dropped": [("run / (1.0 + exp(g[ko * dv + d]))", "run")],
    "logits_chain_rule_sign": [("run / (1.0 + exp(g[ko * dv + d]))", "run / (1.0 + exp(-g[ko * dv + d]))")],
}


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name, builds):
    src = SRC
    for old, new in MUTATIONS[name]:
        assert old in src, f"mutation {name}: pattern not found in the oracle source"
        src = src.replace(old, new)
    c_path = builds / f"{name}.c"
    so_path = builds / f"{name}.so"
    c_path.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-shared", "-fPIC", str(c_path), "-o",
                    str(so_path), "-lm"], check=True)
    lib = O.load(str(so_path))
    failed = []
    for pin, (fn, tol) in ALL_PINS.items():
        try:
            err = fn(lib, np.random.default_rng(1234))
        except (AssertionError, FloatingPointError, RuntimeError):
            failed.append(pin)
            continue
        if not err <= tol:  # NaN counts as a failure
            failed.append(pin)
    assert failed, f"planted mistake '{name}' passed every pin"
