"""Seeded random packs against the oracle, forward and backward.

Each case draws the sample count, the lengths (empty, single tokens, lengths at and
across the 32- and 64-token chunk edges, longer samples), the head count, d_k and d_v,
the data type, q/k normalisation, an initial state and the decay range, so that
combinations the named cases do not list are compared too. Every scan variant the
library picks for those sizes is exercised (the fused scan for bf16 at d_k = d_v = 128,
the two-kernel scan for other bf16 sizes, the sequential kernel for fp32). The scan is
the update of the explainer page ("One stream, three mechanisms, no positions") with the
state reset at each packed sample (paper, Sec. 3 KDA paragraph); the bounds are those of
the named cases.
"""
import numpy as np
import pytest

import gpu_util as gu
from delta_rule_recurrent_kda_amd import inputs
from test_backward_gpu import _compare as bwd_compare
from test_backward_gpu import _draw_grads, _oracle as bwd_oracle, _run as bwd_run

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 5, 31, 32, 33, 63, 64, 65, 100, 257, 700, 1500]


def _case(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 7))
    lens = tuple(int(x) for x in rng.choice(LENGTHS, size=n))
    heads = int(rng.integers(1, 4))
    # half the cases at d_k = d_v = 128, the size of the named workloads
    dk, dv = (128, 128) if rng.random() < 0.5 else (int(rng.choice([64, 128])), int(rng.choice([64, 128])))
    dt = "bf16" if rng.random() < 0.75 else "f32"
    norm = bool(rng.random() < 0.3)
    init = bool(rng.random() < 0.4)
    lar = (float(rng.choice([0.0005, 0.001])), float(rng.choice([0.05, 0.1])))
    return inputs.KdaSpec(f"random{seed}", lens, heads, dk, dv, dt, lar, 9000 + seed), norm, init


def _describe(spec, norm, init):
    return (f"lens={list(spec.seq_lens)} H={spec.heads} dk={spec.dk} dv={spec.dv} {spec.dtype} "
            f"norm={norm} initial_state={init}")


@pytest.mark.parametrize("seed", range(48))
def test_random_pack_forward(seed):
    import torch
    spec, norm, init = _case(seed)
    gu.log(f"case random forward {seed}: {_describe(spec, norm, init)}")
    a = inputs.generate(spec)
    if norm:
        a = gu.unnormalised(spec, a, 50 + seed)
    s0 = None
    if init:
        s0 = (np.random.default_rng(70 + seed).standard_normal(
            (len(spec.seq_lens), spec.heads, spec.dk, spec.dv)) * 0.5).astype(np.float32)
    d = gu.device_inputs(spec, a)
    out, fs = gu.run_hip(spec, d, initial_state=None if s0 is None else torch.from_numpy(s0).to("cuda:0"),
                         qk_l2norm=norm)
    o_ref, f_ref = gu.oracle_ref(spec, a, initial_state=None if s0 is None else s0.astype(np.float64),
                                 qk_l2norm=norm)
    gu.compare(spec, out, fs, o_ref, f_ref, label=f"random forward {seed}")


@pytest.mark.parametrize("seed", range(16))
def test_random_pack_backward(seed):
    spec, norm, init = _case(100 + seed)
    gu.log(f"case random backward {seed}: {_describe(spec, norm, init)}")
    a = inputs.generate(spec)
    if norm:
        a = gu.unnormalised(spec, a, 150 + seed)
    do, dfs, s0 = _draw_grads(spec, 170 + seed)
    if not init:
        dfs = s0 = None
    got = bwd_run(spec, a, do, dfs, s0, norm)
    ref = bwd_oracle(spec, a, do, dfs, s0, norm)
    bwd_compare(spec, got, ref, f"random backward {seed}")
