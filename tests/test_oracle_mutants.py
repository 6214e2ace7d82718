"""Each plausible mistake planted in a copy of the oracle must fail at least one pin.

The copies are built on the CPU from ``oracle/oracle.c`` with one textual change each and
run against ``test_oracle_pins.py`` in a subprocess; the real oracle is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

PINS = "test_oracle_pins.py"
SIG = "test_oracle_sigmoid_pins.py"
PROJ = "test_oracle_projection_pins.py"
BWD = "test_oracle_backward_pins.py"
FWD = "test_oracle_forward_pins.py"

MUTANTS = {
    "tie_to_higher_id": ("if (best < 0 || p[e] > p[best]) best = e;", "if (best < 0 || p[e] >= p[best]) best = e;"),
    "softmax_unnormalised": ("for (int64_t e = 0; e < E; ++e) p[e] /= s;", "(void)s;"),
    "renorm_wrong_terms": ("for (int64_t j = 0; j < k; ++j) den += p[idx[j]];", "for (int64_t j = 0; j < k; ++j) den += p[j];"),
    # (dropping the explicit +inf / all -inf test is not a mistake: the max-subtracted
    # softmax of such rows is NaN everywhere anyway, so that copy is equivalent)
    "nan_row_uniform": ("if (row_softmax(x, E, p)) {\n                for (int64_t j = 0; j < k; ++j) {\n"
                        "                    idx[j] = (uint32_t)j;\n                    store_val(weights, ldt, t * k + j, NAN);",
                        "if (row_softmax(x, E, p)) {\n                for (int64_t j = 0; j < k; ++j) {\n"
                        "                    idx[j] = (uint32_t)j;\n                    store_val(weights, ldt, t * k + j, 1.0 / (double)E);"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_up_swapped": ("hb[r * I + i] = round_to(silu(g) * u, dt);", "hb[r * I + i] = round_to(silu(u) * g, dt);"),
    "down_transposed": ("wd[i] = load_val(down, dt, (e * H + c) * I + i);", "wd[i] = load_val(down, dt, (e * I + i) * H + c);"),
    "combine_one_weight": ("double w = load_val(weights, wdt, t * k + j);\n                    s += w *",
                           "double w = load_val(weights, wdt, t * k);\n                    s += w *"),
    "combine_drops_last": ("for (int64_t j = 0; j < k; ++j) {\n                    double w", "for (int64_t j = 0; j + 1 < k; ++j) {\n                    double w"),
    "dispatch_skips_first": ("for (int64_t a = 0; a < T * k; ++a)\n        if (expert_indices[a]", "for (int64_t a = 1; a < T * k; ++a)\n        if (expert_indices[a]"),
    "rounding_truncates": ("double r = nearbyint(x / q) * q;", "double r = trunc(x / q) * q;"),
    "hidden_not_rounded": ("hb[r * I + i] = round_to(silu(g) * u, dt);", "hb[r * I + i] = silu(g) * u;"),
    # group-limited sigmoid routing (section 10), checked against its own pins
    "sig_bias_in_weights": ("double v = s[idx[j]];", "double v = c[idx[j]];", SIG),
    "sig_expert_tie_to_higher_id": ("if (best < 0 || c[e] > c[best]) best = e;", "if (best < 0 || c[e] >= c[best]) best = e;", SIG),
    "sig_group_tie_to_higher_id": ("if (!gsel[g] && (best < 0 || gs[g] > gs[best])) best = g;",
                                   "if (!gsel[g] && (best < 0 || gs[g] >= gs[best])) best = g;", SIG),
    "sig_top_two_ignored": ("if (!top_two) {\n                    gs[g] = cg[b1];", "if (1) {\n                    gs[g] = cg[b1];", SIG),
    "sig_top_two_counts_max_twice": ("if (i != b1 && (b2 < 0 || cg[i] > cg[b2])) b2 = i;", "if (b2 < 0 || cg[i] > cg[b2]) b2 = i;", SIG),
    "sig_groups_not_enforced": ("if (taken[e] || !gsel[e / per]) continue;", "if (taken[e]) continue;", SIG),
    "sig_scale_dropped_with_renorm": ("v *= scale;", "if (!renormalize) v *= scale;", SIG),
    "sig_nan_row_weights_finite": ("if (nan_row) {\n                for (int64_t j = 0; j < k; ++j) {\n"
                                   "                    idx[j] = (uint32_t)j;\n                    store_val(weights, ldt, t * k + j, NAN);",
                                   "if (nan_row) {\n                for (int64_t j = 0; j < k; ++j) {\n"
                                   "                    idx[j] = (uint32_t)j;\n                    store_val(weights, ldt, t * k + j, 0.0);", SIG),
    # router projection, checked against its own pins
    "proj_router_transposed": ("load_val(router, dt, e * H + h)", "load_val(router, dt, h * E + e)", PROJ),
    "proj_half_the_sum": ("for (int64_t h = 0; h < H; ++h) acc +=", "for (int64_t h = 0; h < H / 2; ++h) acc +=", PROJ),
    "proj_wrong_input_stride": ("load_val(input, dt, t * H + h)", "load_val(input, dt, t * E + h)", PROJ),
    # first-order training, checked against its own pins
    "bwd_quotient_rule_sign": ("(score_partial(sc, scoring, ix[j], e) * S - sc[ix[j]] * dS)",
                               "(score_partial(sc, scoring, ix[j], e) * S + sc[ix[j]] * dS)", BWD),
    "bwd_softmax_partial_index": ("return sc[i] * ((i == e ? 1.0 : 0.0) - sc[e]);",
                                  "return sc[i] * ((i == e ? 1.0 : 0.0) - sc[i]);", BWD),
    "bwd_scale_dropped": ("const double dw = scale * (", "const double dw = (", BWD),
    "bwd_silu_grad_sign": ("return s * (1.0 + z * (1.0 - s));", "return s * (1.0 - z * (1.0 - s));", BWD),
    "bwd_du_without_silu": ("DU[r * I + i] = round_to(dh * silu(g), dt);", "DU[r * I + i] = round_to(dh * g, dt);", BWD),
    "bwd_ddown_from_input": ("sd += DY[r * H + c] * Hh[r * I + i];", "sd += DY[r * H + c] * X[r * H + (i % H)];", BWD),
    "bwd_dx_without_up": ("s += load_val(gate, dt, (e * I + i) * H + c) * DG[r * I + i] +\n                         load_val(up, dt, (e * I + i) * H + c) * DU[r * I + i];",
                          "s += load_val(gate, dt, (e * I + i) * H + c) * DG[r * I + i];", BWD),
    "bwd_dweights_from_weight": ("dw += go * load_val(expert_output, dt, r * H + c);", "dw += go * w;", BWD),
    "bwd_dispatch_skips_last": ("for (int64_t j = 0; j < k; ++j) s += load_val(grad_dispatched",
                                "for (int64_t j = 0; j + 1 < k; ++j) s += load_val(grad_dispatched", BWD),
    # the composed forwards with sigmoid routing and with the gate projection, checked against
    # their own pins
    "fwd_routed_weights_in_token_dtype": ("rc = oracle_combine(y, dt, map, w, ldt, T, k, H, output);\n    if (gate) free(y);\n    free(disp);\n    free(map);\n    free(offs);\n    return rc;",
                                          "rc = oracle_combine(y, dt, map, w, dt, T, k, H, output);\n    if (gate) free(y);\n    free(disp);\n    free(map);\n    free(offs);\n    return rc;", FWD),
    "fwd_routed_combines_the_inputs": ("rc = oracle_combine(y, dt, map, w, ldt, T, k, H, output);\n    if (gate) free(y);\n    free(disp);\n    free(map);\n    free(offs);\n    return rc;",
                                       "rc = oracle_combine(disp, dt, map, w, ldt, T, k, H, output);\n    if (gate) free(y);\n    free(disp);\n    free(map);\n    free(offs);\n    return rc;", FWD),
    "fwd_sigmoid_scale_dropped": ("scale, idx, w, NULL);", "1.0, idx, w, NULL);", FWD),
    "fwd_projected_renorm_dropped": ("oracle_route_projected(input, dt, router, T, H, E, k, renormalize, idx, w, NULL);",
                                     "oracle_route_projected(input, dt, router, T, H, E, k, 0, idx, w, NULL);", FWD),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    old, new, pins = (MUTANTS[name] + (PINS,))[:3]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-w", "-o", str(lib), str(mut), "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
