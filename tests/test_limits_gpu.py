"""The scan at the library's size limit for 32-bit element offsets (GPU).

The limit is total_tokens * num_heads * max(d_k, d_v) < 2^31. The oracle cannot run a pack
that large in test time, so two properties tie the pack to it:
  1. one 1,000-token sample (16 heads, d = 128, bf16) matches the fp64 oracle to the bf16
     tolerance (per output row <= 2e-2 of the row's norm);
  2. a pack of 1,048 copies of that sample (1,048,000 tokens x 16 heads x 128 channels,
     2,146,304,000 elements per tensor) gives, in every copy, the one-sample outputs, final
     states and gradients bit for bit. Samples never exchange data, and each is computed in
     the same order whatever its position in the pack.
The backward's workspace at this size is about 100 GB.
"""
import numpy as np
import pytest

import gpu_util as gu
from delta_rule_recurrent_kda_amd import inputs

pytestmark = pytest.mark.gpu

L1, H, D = 1000, 16, 128


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_scan_at_the_offset_limit():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    N = (2 ** 31 - 1) // (L1 * H * D)
    assert N * L1 * H * D < 2 ** 31 <= (N + 1) * L1 * H * D
    spec = inputs.KdaSpec("limit-one", (L1,), H, D, D, "bf16", (0.001, 0.1), 9191)
    a = inputs.generate(spec)
    d1 = gu.device_inputs(spec, a)
    gu.log(f"case scan at the offset limit: one sample vs the oracle, then {N} copies ({N * L1 * H * D} elements)")
    out1, fs1 = kda.forward(d1["q"], d1["k"], d1["v"], d1["log_alpha"], d1["beta"], d1["cu_seqlens"])
    torch.cuda.synchronize()
    o_ref, f_ref = gu.oracle_ref(spec, a)
    gu.compare(spec, out1.float().cpu().double().numpy(), fs1.cpu().double().numpy(), o_ref, f_ref,
               label="one sample")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(91)
    do1 = torch.randn((L1, H, D), device="cuda:0", generator=g).to(torch.bfloat16)
    grads1 = [t.clone() for t in kda.backward(d1["q"], d1["k"], d1["v"], d1["log_alpha"], d1["beta"],
                                              d1["cu_seqlens"], do1) if t is not None]
    torch.cuda.synchronize()

    rep = lambda t: t.repeat(N, *([1] * (t.dim() - 1)))
    q, k, v, la, b = (rep(d1[n]) for n in ("q", "k", "v", "log_alpha", "beta"))
    cu = torch.arange(N + 1, dtype=torch.int32, device="cuda:0") * L1
    out, fs = kda.forward(q, k, v, la, b, cu)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out).view(N, L1, H, D), _bits(out1).unsqueeze(0).expand(N, L1, H, D))
    assert torch.equal(_bits(fs), _bits(fs1).expand(N, H, D, D))
    del out, fs
    do = rep(do1)
    grads = [t for t in kda.backward(q, k, v, la, b, cu, do) if t is not None]
    torch.cuda.synchronize()
    for x, y in zip(grads, grads1):
        if x.shape[0] == N:                     # per-sample gradients (d_initial_state)
            assert torch.equal(_bits(x), _bits(y).expand_as(x))
        else:                                   # per-token gradients
            shape = (N, L1) + tuple(x.shape[1:])
            assert torch.equal(_bits(x).view(shape), _bits(y).unsqueeze(0).expand(shape))
