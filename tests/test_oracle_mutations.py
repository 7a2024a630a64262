"""Plausible mistakes planted in a copy of the oracle source must be caught.

Each mutation rewrites one expression of a temporary copy of the C source
(never the committed file), compiles it on the CPU, and runs the pin checks
against it.  At least one pin must exceed its tolerance by a wide margin;
otherwise the pins would not protect the oracle from that kind of mistake.
"""
import os

import pytest

import oracle
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "wkv7_oracle.c")

# (name, text in the source, replacement)
MUTATIONS = [
    ("sa_uses_b", "acc += S[i * D + j] * at[j];", "acc += S[i * D + j] * bt[j];"),
    ("drop_vk", "+ vt[i] * kt[j] + sa[i] * bt[j];", "+ sa[i] * bt[j];"),
    ("transposed_vk", "+ vt[i] * kt[j] + sa[i] * bt[j];", "+ vt[j] * kt[i] + sa[i] * bt[j];"),
    ("sa_sign", "+ vt[i] * kt[j] + sa[i] * bt[j];", "+ vt[i] * kt[j] - sa[i] * bt[j];"),
    ("decay_on_row", "S[i * D + j] = wt[j] * S[i * D + j]", "S[i * D + j] = wt[i] * S[i * D + j]"),
    ("y_transposed", "for (int j = 0; j < D; ++j) acc += S[i * D + j] * rt[j];",
     "for (int j = 0; j < D; ++j) acc += S[j * D + i] * rt[j];"),
    ("ckpt_after_chunk", "if (J->ckpt && t % ORACLE_CHUNK == 0) {",
     "if (J->ckpt && t % ORACLE_CHUNK == 1) {"),
    ("dr_uses_prev_state", "acc += dyt[i] * St[i * D + j];", "acc += dyt[i] * Sp[i * D + j];"),
    ("dw_before_b2", "aw += g[i * D + j] * Sp[i * D + j];", "aw += (g[i * D + j] - dyt[i] * rt[j]) * Sp[i * D + j];"),
    ("dk_uses_k", "ak += g[i * D + j] * vt[i];", "ak += g[i * D + j] * kt[i];"),
    ("db_sign", "dbt[j] = ab;", "dbt[j] = -ab;"),
    ("dv_uses_b", "av += g[i * D + j] * kt[j];", "av += g[i * D + j] * bt[j];"),
    ("da_uses_state_t", "for (int i = 0; i < D; ++i) acc += dsa[i] * Sp[i * D + j];",
     "for (int i = 0; i < D; ++i) acc += dsa[i] * St[i * D + j];"),
    ("g_carry_drops_a", "g[i * D + j] = wt[j] * g[i * D + j] + dsa[i] * at[j];",
     "g[i * D + j] = wt[j] * g[i * D + j];"),
    ("g_carry_uses_b", "g[i * D + j] = wt[j] * g[i * D + j] + dsa[i] * at[j];",
     "g[i * D + j] = wt[j] * g[i * D + j] + dsa[i] * bt[j];"),
    ("dhT_ignored", "if (J->dhT) memcpy(g,", "if (0) memcpy(g,"),
    ("proj_w_sign", "w[o + j] = exp(-c * logistic(w_raw[o + j]));", "w[o + j] = exp(c * logistic(w_raw[o + j]));"),
    ("proj_w_no_scale", "w[o + j] = exp(-c * logistic(w_raw[o + j]));", "w[o + j] = exp(-logistic(w_raw[o + j]));"),
    ("proj_a_sign", "a[o + j] = -kh;", "a[o + j] = kh;"),
    ("proj_b_ungated", "b[o + j] = kh * logistic(alpha[o + j]);", "b[o + j] = kh;"),
    ("proj_b_gate_flipped", "b[o + j] = kh * logistic(alpha[o + j]);", "b[o + j] = kh * logistic(-alpha[o + j]);"),
    ("proj_norm_squared", "const double n = sqrt(nn);\n        for (int j = 0; j < D; ++j) {\n            const double kh",
     "const double n = nn;\n        for (int j = 0; j < D; ++j) {\n            const double kh"),
    ("proj_dw_raw_sign", "dw_raw[o + j] = dw[o + j] * wj * (-c) * sw * (1.0 - sw);",
     "dw_raw[o + j] = dw[o + j] * wj * c * sw * (1.0 - sw);"),
    ("proj_dw_raw_no_w", "dw_raw[o + j] = dw[o + j] * wj * (-c) * sw * (1.0 - sw);",
     "dw_raw[o + j] = dw[o + j] * (-c) * sw * (1.0 - sw);"),
    ("proj_g_sign", "const double g = -da[o + j] + db[o + j] * sa;", "const double g = da[o + j] + db[o + j] * sa;"),
    ("proj_dalpha_no_kh", "dalpha[o + j] = db[o + j] * kh * sa * (1.0 - sa);",
     "dalpha[o + j] = db[o + j] * sa * (1.0 - sa);"),
    ("proj_dkappa_no_projection", "dkappa[o + j] = n > 0.0 ? (g - kh * proj) / n : 0.0;",
     "dkappa[o + j] = n > 0.0 ? g / n : 0.0;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    bad = tmp_path / f"mut_{name}.c"
    bad.write_text(src.replace(old, new))
    lib = oracle.OracleLib(oracle.compile_source(str(bad), str(tmp_path / f"mut_{name}.so")))
    worst = 0.0
    for check, fn in pins.ALL.items():
        try:
            ratio = fn(lib) / pins.TOL[check]
        except Exception:   # a crash or shape error also counts as caught
            ratio = float("inf")
        if ratio != ratio:  # NaN
            ratio = float("inf")
        worst = max(worst, ratio)
        if worst > 1e3:
            break
    assert worst > 1e3, f"mutation {name} slipped through every pin (worst ratio {worst:.2e})"
