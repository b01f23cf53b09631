"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, a wrong index, a transposed
operand) in a private copy of the oracle's C source, builds it into a temporary library on the
CPU, and checks that at least one pin fails on it. The real oracle is never modified.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("prediction_not_decayed", "e[c] = vv[c] - a * p[c];", "e[c] = vv[c] - p[c];"),
    ("write_sign", "Sr[c] = a * Sr[c] + bk * e[c];", "Sr[c] = a * Sr[c] - bk * e[c];"),
    ("no_state_decay", "Sr[c] = a * Sr[c] + bk * e[c];", "Sr[c] = Sr[c] + bk * e[c];"),
    ("interleaved_head_map", "const int h = j * G + gi;\n    init_state(J, n, h, S);\n    for (int64_t t = 0; t < L; ++t) {\n      const int64_t tau = t0 + t;\n      load_row(J->q",
     "const int h = gi * J->H + j;\n    init_state(J, n, h, S);\n    for (int64_t t = 0; t < L; ++t) {\n      const int64_t tau = t0 + t;\n      load_row(J->q"),
    ("no_l2norm_scale", "for (int i = 0; i < d; ++i) out[i] *= r;", "(void)r;"),
    ("bwd_dalpha_drops_p_term", "dalpha -= p[c] * de[c];", "(void)0;"),
    ("bwd_dk_drops_state_term", "dk_t[r] += b * dSe[r] + s;", "dk_t[r] += b * dSe[r];"),
    ("bwd_dS_drops_rank1", "dSr[c] = a * dSr[c] + kh[r] * dp[c];", "dSr[c] = a * dSr[c];"),
    ("bwd_dg_missing_chain", "J->dg[(size_t)tau * J->HV + h] = a * dalpha;", "J->dg[(size_t)tau * J->HV + h] = dalpha;"),
    ("bwd_norm_drops_projection", "out[r] = (dxh[r] - qh[r] * dot) * r_inv;", "out[r] = dxh[r] * r_inv;"),
    ("bwd_dq_uses_old_state", "const double* Scr = Sc + (size_t)r * dv;", "const double* Scr = Sp + (size_t)r * dv;"),
    ("bwd_dv_sign", "for (int c = 0; c < dv; ++c) out[c] = de[c];", "for (int c = 0; c < dv; ++c) out[c] = -de[c];"),
    ("bwd_dbeta_dropped", "dbeta += kh[r] * s;", "(void)0;"),
    ("bwd_ignores_dht", "if (J->dht) {", "if (0) {"),
    ("bwd_beta_in_de_dropped", "de[c] = b * tmp[c];", "de[c] = tmp[c];"),
    ("chunked_decay_reversed", "(i > jj) ? bet[i] * exp(Gc[i] - Gc[jj]) * sk : 0.0;", "(i > jj) ? bet[i] * exp(Gc[jj] - Gc[i]) * sk : 0.0;"),
    ("chunked_strict_output_mask", "(i >= jj) ? exp(Gc[i] - Gc[jj]) * sq : 0.0;", "(i > jj) ? exp(Gc[i] - Gc[jj]) * sq : 0.0;"),
    ("chunked_no_gamma", "S[(size_t)r * dv + c] = gam * S[(size_t)r * dv + c] + s;", "S[(size_t)r * dv + c] = S[(size_t)r * dv + c] + s;"),
    ("chunked_transposed_kk", "sk += Kh[(size_t)i * dk + r] * Kh[(size_t)jj * dk + r];", "sk += Kh[(size_t)i * dk + r] * Qh[(size_t)jj * dk + r];"),
]


def _build_mutant(tmpdir, find, repl):
    src = open(SRC).read()
    assert src.count(find) >= 1, "mutation anchor not found: %r" % find
    mutated = src.replace(find, repl, 1)
    path = os.path.join(tmpdir, "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    out = os.path.join(tmpdir, "libmutant.so")
    oracle.build(path, out)
    return oracle.load(out)


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, find, repl):
    with tempfile.TemporaryDirectory() as d:
        lib = _build_mutant(d, find, repl)
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib)
            except (AssertionError, RuntimeError, FloatingPointError):
                caught.append(pin.__name__)
        assert caught, "no pin catches the planted mistake %s" % name
