"""The fp64 short-convolution oracle against textbook and library routines, shifts and
invariants; planted mistakes must be caught (CPU only)."""
import os
import subprocess

import pytest

import pins_conv

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "short_conv_oracle.c")


@pytest.mark.parametrize("pin", pins_conv.ALL_CONV_PINS, ids=lambda p: p.__name__)
def test_short_conv_oracle_pin(oracle_mod, pin):
    pin(oracle_mod.short_conv)


MUTANTS = {
    "time_not_causal": ("const int64_t ii = i - a,", "const int64_t ii = i + a,"),
    "space_not_centred": ("jj = j + b - ph,", "jj = j + b,"),
    "text_kernel_reversed": ("acc += w_text[(int64_t)i * C + c]", "acc += w_text[(int64_t)(kx - 1 - i) * C + c]"),
    "height_width_weights_swapped": ("w_vis[(((int64_t)a * kh + b) * kw + d) * C + c]",
                                     "w_vis[(((int64_t)a * kw + d) * kh + b) * C + c]"),
    "text_reads_future_tokens": ("if (t - i >= 0) acc +=", "if (t - i >= 0 && t + i < L) acc += 0.5 * x[(base + t + i) * C + c] * w_text[(int64_t)i * C + c] +"),
    "no_time_taps": ("for (int32_t a = 0; a < kt; ++a)", "for (int32_t a = 0; a < 1; ++a)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_short_conv_mutant_is_caught(tmp_path, oracle_mod, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c)], check=True)
    conv = oracle_mod.kda_oracle.short_conv_from(str(so))
    caught = []
    for pin in pins_conv.ALL_CONV_PINS:
        try:
            pin(conv)
        except (AssertionError, ValueError, RuntimeError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
