"""Plant plausible mistakes in a copy of the oracle's C source and check that
every one of them is caught by at least one pin (CPU only, compiled with gcc)."""
import os
import subprocess

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kda_oracle.c")

MUTANTS = {
    "no_decay": ("row[j] *= a;", "row[j] *= 1.0;"),
    "inverted_gate": ("const double a = exp(lat[c]);", "const double a = exp(-lat[c]);"),
    "erase_sign": ("u[j] = bt * (vt[j] - p[j]);", "u[j] = bt * (vt[j] + p[j]);"),
    "no_erase_linear_attention": ("u[j] = bt * (vt[j] - p[j]);", "u[j] = bt * vt[j];"),
    "beta_on_write_only": ("u[j] = bt * (vt[j] - p[j]);", "u[j] = bt * vt[j] - p[j];"),
    "no_reset": ("const int64_t t0 = job->cu_seqlens[n], t1", "const int64_t t0 = 0, t1"),
    "readout_key_not_query": ("const double qc = qt[c];", "const double qc = kt[c];"),
    "initial_state_ignored": ("    if (job->initial_state)\n", "    if (0)\n"),
    "qk_norm_ignored": ("if (job->qk_l2norm) {", "if (0) {"),
    "qk_norm_query_only": ("            qt = qn;\n            kt = kn;\n", "            qt = qn;\n"),
    "qk_norm_squared_length": ("sk = sk > 0.0 ? 1.0 / sqrt(sk) : 0.0;", "sk = sk > 0.0 ? 1.0 / sk : 0.0;"),
    "qk_norm_key_by_query_length": ("kn[c] = kt[c] * sk;", "kn[c] = kt[c] * sq;"),
    "decay_after_retrieve": (
        "        /* u = beta_t (v_t - p) */\n",
        "        for (int32_t c = 0; c < dk; ++c) for (int32_t j = 0; j < dv; ++j) p[j] += 0.0 * c;\n"
        "        for (int32_t j = 0; j < dv; ++j) { double s = 0; for (int32_t c = 0; c < dk; ++c)"
        " s += S[(size_t)c * dv + j] / exp(lat[c]) * kt[c]; p[j] = s; }\n"
        "        /* u = beta_t (v_t - p) */\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, oracle_mod, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c), "-lm",
                    "-lpthread"], check=True)
    fwd = oracle_mod.kda_oracle.forward_from(str(so))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
