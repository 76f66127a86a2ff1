"""The fp64 reverse-mode oracle against finite differences of the pinned forward and
against autograd of the dense formulation; planted mistakes must be caught (CPU only)."""
import os
import subprocess

import pytest

import pins_bwd

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kda_oracle.c")


@pytest.mark.parametrize("pin", pins_bwd.ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(oracle_mod, pin):
    pin(oracle_mod.forward, oracle_mod.backward)


MUTANTS = {
    "no_erase_term_in_state_grad": ("dSt[(size_t)c * dv + j] = dS[(size_t)c * dv + j] + kn[c] * dp[j];",
                                    "dSt[(size_t)c * dv + j] = dS[(size_t)c * dv + j];"),
    "retrieve_grad_sign": ("dp[j] = -bt * du[j];", "dp[j] = bt * du[j];"),
    "no_decay_on_carried_grad": ("dS[(size_t)c * dv + j] = a * dSt[(size_t)c * dv + j];",
                                 "dS[(size_t)c * dv + j] = dSt[(size_t)c * dv + j];"),
    "gate_grad_misses_erase": ("acc += dSt[(size_t)c * dv + j] * St[(size_t)c * dv + j];",
                               "acc += dS[(size_t)c * dv + j] * St[(size_t)c * dv + j];"),
    "readout_grad_from_previous_state": (
        "acc += S[(size_t)c * dv + j] * dot[j];",
        "acc += prev[(size_t)(t - b0) * SS + (size_t)c * dv + j] * dot[j];"),
    "beta_grad_misses_retrieval": ("db += du[j] * (vt[j] - p[j]);", "db += du[j] * vt[j];"),
    "norm_grad_without_projection": ("dqt[c] = (dqn[c] - qn[c] * sq) * qinv;", "dqt[c] = dqn[c] * qinv;"),
    "key_grad_misses_retrieval": ("                dkn[c] += acc;\n", "                dkn[c] += 0.0 * acc;\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(tmp_path, oracle_mod, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c), "-lm",
                    "-lpthread"], check=True)
    fwd = oracle_mod.kda_oracle.forward_from(str(so))
    bwd = oracle_mod.kda_oracle.backward_from(str(so))
    caught = []
    for pin in pins_bwd.ALL_BWD_PINS:
        try:
            pin(fwd, bwd)
        except (AssertionError, ValueError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
