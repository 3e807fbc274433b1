"""Planted mistakes in the CPU oracle must be caught by the pins (no GPU).

Each mutant is a copy of ``oracle.c`` with one plausible slip (a dropped
term, a wrong sign or index, an off-by-one window, swapped operands),
compiled into a temporary directory; the test runs every pin of
``oracle_pins`` against it and requires at least one to fail.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle
from tests import oracle_pins

MUTANTS = {
    "gate_swapped": ("*g = 1.0 / (1.0 + exp(-logit));", "*g = 1.0 / (1.0 + exp(logit));"),
    "gbar_is_one": ("*gbar = 1.0 / (1.0 + exp(logit));", "*gbar = 1.0;"),
    "restart_offset": ("if (!full && t % L == 0)", "if (!full && t % L == 1)"),
    "restart_dropped": ("if (!full && t % L == 0) { hk = 0.0; hv = 0.0; }", ""),
    "recurrence_input_ungated": ("hk = g * hk + gb * k[i];", "hk = g * hk + k[i];"),
    "value_uses_key": ("hv = g * hv + gb * v[i];", "hv = g * hv + gb * k[i];"),
    "sliding_window_too_long": ("int lo = t - L + 1;", "int lo = t - L;"),
    "sliding_product_order": ("hk += prod * gb * k[i];\n                            hv += prod * gb * v[i];\n                            prod *= g;",
                              "prod *= g;\n                            hk += prod * gb * k[i];\n                            hv += prod * gb * v[i];"),
    "dilated_skips_own_state": ("for (int s = t; s >= 0; s -= D) {\n        kp[n]",
                                "for (int s = t - D; s >= 0; s -= D) {\n        kp[n]"),
    "dilated_stride_off_by_one": ("for (int s = t; s >= 0; s -= D) {\n        kp[n]",
                                  "for (int s = t; s >= 0; s -= D + 1) {\n        kp[n]"),
    "local_window_short": ("for (int w = 0; w < W && t - w >= 0; ++w) {\n        kp[n]",
                           "for (int w = 0; w + 1 < W && t - w >= 0; ++w) {\n        kp[n]"),
    "local_window_shifted": ("kp[n] = kr + idx4(b, t - w, h, 0, T, H, d);\n        vp[n] = vr + idx4(b, t - w, h, 0, T, H, d);",
                             "kp[n] = kr + idx4(b, t - w > 0 ? t - w - 1 : 0, h, 0, T, H, d);\n        vp[n] = vr + idx4(b, t - w > 0 ? t - w - 1 : 0, h, 0, T, H, d);"),
    "local_uses_states": ("kp[n] = kr + idx4(b, t - w, h, 0, T, H, d);",
                          "kp[n] = ks + idx4(b, t - w, h, 0, T, H, d);"),
    "scale_dropped": ("z[j] = scale * dot;", "z[j] = dot;"),
    "softmax_sign": ("double w = exp(z[j] - m);", "double w = exp(m - z[j]);"),
    "softmax_unnormalised": ("for (int c = 0; c < d; ++c) out[c] /= den;", ""),
    "qk_transposed_index": ("for (int c = 0; c < d; ++c) dot += q[c] * keys[j][c];",
                            "for (int c = 0; c < d; ++c) dot += q[c] * keys[j][d - 1 - c];"),
    "decode_count_floor": ("int nd = (T - 1) / D[h] + 1;\n                    int nw",
                           "int nd = T / D[h];\n                    int nw"),
    "decode_ring_short": ("for (int j = 0; j < nw; ++j) {", "for (int j = 0; j + 1 < nw; ++j) {"),
    "chunk_end_off_by_one": ("for (int p = D - 1; p < t; p += D) {", "for (int p = D; p < t; p += D) {"),
    "chunk_end_not_strict": ("for (int p = D - 1; p < t; p += D) {", "for (int p = D - 1; p <= t; p += D) {"),
    "chunk_own_state_dropped": ("    if (pos) pos[n] = t;\n    return n + 1;", "    return n;"),
    "bwd_delta_dropped": ("double ds = p[j] * (z[j] - delta);", "double ds = p[j] * z[j];"),
    "bwd_gate_derivative_sign": ("dlogit[i] = g * gb * (", "dlogit[i] = -g * gb * ("),
    "bwd_restart_carry_kept": ("lk = cut ? 0.0 : g * lamk;", "lk = g * lamk;"),
    "bwd_input_grad_ungated": ("dk[i] += gb * lamk;", "dk[i] += lamk;"),
    "bwd_raw_path_to_states": ("kp[nk] = k + o; vp[nk] = v + o; dkp[nk] = dk + o; dvp[nk] = dv + o;",
                               "kp[nk] = k + o; vp[nk] = v + o; dkp[nk] = dks + o; dvp[nk] = dvs + o;"),
    "bwd_prev_state_off_by_one": ("double hv_prev = cut ? 0.0 : vs[idx4(b, t - 1, h, c, T, H, d)];",
                                  "double hv_prev = cut ? 0.0 : vs[idx4(b, t, h, c, T, H, d)];"),
    "bwd_sliding_window_long": ("const int lo = t - L + 1 < 0 ? 0 : t - L + 1;\n                                double g, gb;",
                                "const int lo = t - L < 0 ? 0 : t - L;\n                                double g, gb;"),
    "bwd_sliding_suffix_shifted": ("Q[u - 1 - lo] = Q[u - lo] * g;", "Q[u - 1 - lo] = Q[u - lo];"),
    "bwd_sliding_state_after_step": ("dlogit[i] += g * gb * (qk * (wk - k[i]) + qv * (wv - v[i]));\n                                    wk = g * wk + gb * k[i];\n                                    wv = g * wv + gb * v[i];",
                                     "wk = g * wk + gb * k[i];\n                                    wv = g * wv + gb * v[i];\n                                    dlogit[i] += g * gb * (qk * (wk - k[i]) + qv * (wv - v[i]));"),
    "count_window_short": ("for (int w = 0; w < W && t - w >= 0; ++w) {\n        if (loc)",
                           "for (int w = 1; w < W && t - w >= 0; ++w) {\n        if (loc)"),
    # the backward at given states: states handed over swapped, or the gate
    # term reading the state at t instead of t - 1
    "bwd_states_swapped": ("oracle_layer_backward_states(q, k, v, logit, ks, vs, dout,",
                           "oracle_layer_backward_states(q, k, v, logit, vs, ks, dout,"),
    "bwd_states_prev_is_current": ("double hv_prev = cut ? 0.0 : vs[idx4(b, t - 1, h, c, T, H, d)];",
                                   "double hv_prev = cut ? 0.0 : vs[idx4(b, t, h, c, T, H, d)];"),
}


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Runs every pin on one compiled mutant in a child process (a mutant may
# also crash outright, e.g. by overrunning a key buffer: that counts as
# caught too) and prints the names of the pins that failed.
_RUNNER = """
import sys
sys.path.insert(0, {root!r})
from oracle import oracle
from tests import oracle_pins
o = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    try:
        pin(o)
    except Exception:
        print("FAILED", pin.__name__, flush=True)
"""


def _caught_by(lib):
    env = dict(os.environ, OMP_NUM_THREADS="2")
    proc = subprocess.run([sys.executable, "-c", _RUNNER.format(root=ROOT, lib=lib)],
                          capture_output=True, text=True, timeout=300, env=env)
    if proc.returncode != 0:
        return [f"crashed({proc.returncode})"]
    return [line.split()[1] for line in proc.stdout.splitlines() if line.startswith("FAILED")]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    with open(oracle.SOURCE) as f:
        src = f.read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site of {name} not unique"
    path = os.path.join(tmp_path, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.compile_oracle(path, os.path.join(tmp_path, f"lib{name}.so"))
    caught = _caught_by(lib)
    assert caught, f"no pin catches the planted mistake {name}"
