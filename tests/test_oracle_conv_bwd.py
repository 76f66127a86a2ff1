"""The fp64 reverse mode of the short convolution against the transposes of the pinned
forward (adjoint identities, dense brute force) and modality separation; planted mistakes
must be caught (CPU only)."""
import os
import subprocess

import pytest

import pins_conv_bwd

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "short_conv_oracle.c")


@pytest.mark.parametrize("pin", pins_conv_bwd.ALL_CONV_BWD_PINS, ids=lambda p: p.__name__)
def test_short_conv_backward_oracle_pin(oracle_mod, pin):
    pin(oracle_mod.short_conv, oracle_mod.short_conv_backward)


MUTANTS = {
    "dx_without_weight": ("dx[src] += w_vis[wi] * g;", "dx[src] += g;"),
    "dw_vis_from_output_position": ("dw_vis[wi] += x[src] * g;",
                                    "dw_vis[wi] += x[(v0 + (i * H + j) * W + k) * C + c] * g;"),
    "text_dx_to_output_token": ("dx[(base + t - ti) * C + c] += w_text", "dx[(base + t) * C + c] += w_text"),
    "time_taps_reversed": ("const int64_t wi = (((int64_t)ta * kh + tb)", "const int64_t wi = (((int64_t)(kt - 1 - ta) * kh + tb)"),
    "first_text_tap_dropped": ("for (int32_t ti = 0; ti < kx; ++ti)", "for (int32_t ti = 1; ti < kx; ++ti)"),
    "space_flipped": ("sj = j + tb - ph,", "sj = j - tb + ph,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_short_conv_backward_mutant_is_caught(tmp_path, oracle_mod, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c)], check=True)
    conv_bwd = oracle_mod.kda_oracle.short_conv_backward_from(str(so))
    caught = []
    for pin in pins_conv_bwd.ALL_CONV_BWD_PINS:
        try:
            pin(oracle_mod.short_conv, conv_bwd)
        except (AssertionError, ValueError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
