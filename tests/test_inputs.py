"""Seeded input generator: reproducibility, shapes, rounding (CPU only)."""
import json
import math
import os
import struct

import numpy as np
import pytest

from delta_rule_recurrent_kda_amd import inputs


def _bf16_rne_scalar(x: float) -> int:
    """Nearest-even bf16 of an fp64 value, from the exact binary expansion."""
    if math.isnan(x):
        return 0x7FC0
    if x == 0:
        return 0x8000 if math.copysign(1, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    m, e = math.frexp(a)              # a = m * 2^e, 0.5 <= m < 1
    e -= 1                            # a = (2m) * 2^e with 1 <= 2m < 2
    if e < -126:                      # subnormal bf16: quantum 2^-133
        q = a / 2.0 ** -133
    else:
        q = a / 2.0 ** (e - 7)        # 8 significant bits incl. the hidden one
    lo = math.floor(q)
    r = q - lo
    n = lo + (1 if (r > 0.5 or (r == 0.5 and lo % 2 == 1)) else 0)
    val = n * (2.0 ** -133 if e < -126 else 2.0 ** (e - 7))
    f32 = struct.unpack("<I", struct.pack("<f", val))[0] if val < 3.4e38 else 0x7F800000
    return sign | (f32 >> 16)


def test_bf16_rounding_matches_scalar_definition():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(2000), rng.uniform(-1e-3, 1e-3, 500),
                         -rng.uniform(0.0005, 0.1, 500)])
    # exact ties and near-ties of the 8-bit significand
    base = np.array([1.0 + (2 * i + 1) * 2.0 ** -8 for i in range(50)])
    xs = np.concatenate([xs, base, -base, base + 2.0 ** -40, base - 2.0 ** -40, [0.0, -0.0, 1e-40]])
    got = inputs.f64_to_bf16_bits(xs)
    want = np.array([_bf16_rne_scalar(float(x)) for x in xs], np.uint16)
    assert np.array_equal(got, want)
    back = inputs.bf16_bits_to_f64(got)
    normal = np.abs(xs) > 1e-30
    assert np.all(np.abs(back - xs)[normal] <= np.abs(xs)[normal] * 2.0 ** -8)


def test_double_rounding_case_is_avoided():
    # fp32 RNE of this value lands exactly on a bf16 tie and would round up; the
    # correctly rounded bf16 is the lower neighbour
    x = 1.0 + 2.0 ** -8 - 2.0 ** -30
    assert inputs.f64_to_bf16_bits(np.array([x]))[0] == _bf16_rne_scalar(x) == 0x3F80


def test_packed_lengths_rule():
    seed, lens = inputs._packed_lengths_seed_rule()
    assert seed == 1003
    assert lens == [1576, 1185, 2602, 1432, 1527, 2285, 3621, 2880]
    assert sum(lens) == 17108


@pytest.mark.parametrize("cfg,T,H,d,dtype", [(0, 1024, 1, 64, "f32"), (1, 17108, 16, 128, "bf16"),
                                             (2, 17408, 16, 128, "bf16"), (3, 33272, 16, 128, "bf16"),
                                             (4, 189272, 16, 128, "bf16")])
def test_config_shapes(cfg, T, H, d, dtype):
    s = inputs.config(cfg)
    assert s.total_tokens == T and s.heads == H and s.dk == s.dv == d and s.dtype == dtype
    cu = s.cu_seqlens()
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    if s.grid is not None:
        Tg, Hg, Wg = s.grid
        assert s.seq_lens[0] == s.text_tokens[0] + Tg * Hg * Wg


def test_generation_reproducible_and_distributed():
    s = inputs.custom([300, 200], heads=3, d=64, dtype="bf16", seed=7)
    a = inputs.generate(s)
    b = inputs.generate(s)
    for key in a:
        assert np.array_equal(a[key], b[key])
    # a single head slice regenerates alone
    c = inputs.generate(s, heads=[1])
    assert np.array_equal(c["k"][:, 1], a["k"][:, 1]) and not c["k"][:, 0].any()
    k = inputs.to_f64(a["k"], "bf16")
    assert np.allclose(np.linalg.norm(k, axis=2), 1.0, atol=3e-3)
    la = inputs.to_f64(a["log_alpha"], "bf16")
    assert la.max() < 0 and la.min() > -0.101
    beta = inputs.to_f64(a["beta"], "bf16")
    assert 0 < beta.min() and beta.max() < 1


def test_f32_unit_norm():
    s = inputs.config(0)
    a = inputs.generate(s)
    assert a["q"].dtype == np.float32
    assert np.allclose(np.linalg.norm(a["q"].astype(np.float64), axis=2), 1.0, atol=1e-6)


def test_raster_order_golden():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "raster_order.json")))
    T, H, W = g["grid"]
    grid = np.arange(T * H * W).reshape(T, H, W)
    flat = grid.reshape(-1)                      # C-order flattening is the scan order
    for (i, j, k), m in g["cases"]:
        assert inputs.raster_index(i, j, k, H, W) == m
        assert flat[m] == grid[i, j, k]
