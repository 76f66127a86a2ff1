"""GPU parity of kda_backward (through the C ABI) against the fp64 reverse-mode oracle.

Two checks per gradient tensor:
- per (sample, head) block, the relative Frobenius norm of the difference: fp32 data 1e-4
  (the arithmetic is fp32 throughout); bf16 data 1e-2 (inputs, d_out and the gradients are
  bf16; one rounding of a gradient to bf16 alone gives about 1.7e-3 on such blocks);
- per row: for dq, dk, dv and dlog_alpha each (token, head) row over its channels, for
  d_initial_state each key-channel row of each (sample, head) state, the largest absolute
  error is at most ROW_TOL times that row's scale; dbeta has one value per (token, head),
  its row is the value itself. A row's scale is its oracle norm, floored at ROW_FLOOR times
  the root mean square of the row norms of its (sample, head) block: some rows are exactly
  zero (dlog_alpha at the first token of a sample that starts from a zero state: the decay
  acts on a zero state) or near-cancelling sums (single dbeta values), and have no relative
  error of their own to speak of; the floor still fails a row that is wrong by more than a
  small fraction of its neighbours' size. A block that is exactly zero as a whole (dlog_alpha
  of a one-token sample from a zero state) takes the root mean square over all rows of its
  head instead: the kernel forms it from sums of terms of that size. The first token of every sample is reported
  separately: a wrong reset or boundary shows there first.
"""
import numpy as np
import pytest

import gpu_util as gu
from delta_rule_recurrent_kda_amd import inputs

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "d_initial_state")
# per-row bounds: bf16 storage rounds each element to 2^-8 relative (RNE), so a row's largest
# element error from the storage alone is at most 2^-8 of its largest element; 2e-2 of the row
# norm (the forward's bound) leaves room for the fp32 arithmetic. fp32 data: 1e-3.
ROW_TOL = {"bf16": 2e-2, "f32": 1e-3}
ROW_FLOOR = 0.05


def _draw_grads(spec, seed):
    rng = np.random.default_rng(seed)
    T, H, N = spec.total_tokens, spec.heads, len(spec.seq_lens)
    do = rng.standard_normal((T, H, spec.dv))
    do = inputs.f64_to_bf16_bits(do) if spec.dtype == "bf16" else do.astype(np.float32)
    dfs = (rng.standard_normal((N, H, spec.dk, spec.dv)) * 0.5).astype(np.float32)
    s0 = (rng.standard_normal((N, H, spec.dk, spec.dv)) * 0.5).astype(np.float32)
    return do, dfs, s0


def _run(spec, a, do, dfs, s0, norm):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    d = gu.device_inputs(spec, a)
    dev = "cuda:0"
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    tdo = (torch.from_numpy(do.view(np.int16)).view(torch.bfloat16) if spec.dtype == "bf16"
           else torch.from_numpy(do)).to(dev)
    assert tdo.dtype == dt
    g = kda.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"], tdo,
                     d_final_state=None if dfs is None else torch.from_numpy(dfs).to(dev),
                     initial_state=None if s0 is None else torch.from_numpy(s0).to(dev),
                     qk_l2norm=norm)
    torch.cuda.synchronize()
    return [x.float().cpu().double().numpy() for x in g]


def _oracle(spec, a, do, dfs, s0, norm):
    import oracle
    f = {x: inputs.to_f64(a[x], spec.dtype) for x in ("q", "k", "v", "log_alpha", "beta")}
    return oracle.backward(f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], a["cu_seqlens"],
                           inputs.to_f64(do, spec.dtype), dfs, s0, qk_l2norm=norm,
                           threads=16)


def _row_errors(name, x, y, cu):
    """Per-row relative errors of one gradient tensor (see the module docstring), and the mask
    of rows that are the first token of a sample."""
    if name == "d_initial_state":
        e = np.abs(x - y).max(axis=3)
        n = np.linalg.norm(y, axis=3)
        return np.where(n > 0, e / np.where(n > 0, n, 1.0), np.where(e > 0, np.inf, 0.0)), None
    first = np.zeros(x.shape[0], bool)
    first[[c for c, c1 in zip(cu[:-1], cu[1:]) if c1 > c]] = True
    if name == "dbeta":
        e, norm = np.abs(x - y), np.abs(y)
    else:
        e, norm = np.abs(x - y).max(axis=2), np.linalg.norm(y, axis=2)
    scale = norm.copy()
    head_rms = np.sqrt(np.mean(norm ** 2, axis=0)) if norm.size else 0.0
    for n0, n1 in zip(cu[:-1], cu[1:]):
        if n1 > n0:
            rms = np.sqrt(np.mean(norm[n0:n1] ** 2, axis=0))
            rms = np.where(rms > 0, rms, head_rms)     # a block that is exactly zero
            scale[n0:n1] = np.maximum(norm[n0:n1], ROW_FLOOR * rms)
    rel = np.where(scale > 0, e / np.where(scale > 0, scale, 1.0), np.where(e > 0, np.inf, 0.0))
    return rel, first


def _compare(spec, got, ref, label):
    tol = 1e-4 if spec.dtype == "f32" else 1e-2
    row_tol = ROW_TOL[spec.dtype]
    cu = spec.cu_seqlens()
    worst, rows = {}, {}
    for name, x, y in zip(NAMES, got, ref):
        w = 0.0
        for n in range(len(cu) - 1):
            for h in range(spec.heads):
                if name == "d_initial_state":
                    a, b = x[n, h], y[n, h]
                else:
                    a, b = x[cu[n]:cu[n + 1], h], y[cu[n]:cu[n + 1], h]
                if b.size == 0:
                    continue
                nb = np.linalg.norm(b)
                e = np.linalg.norm(a - b) / nb if nb > 0 else np.abs(a).max()
                w = max(w, e)
        worst[name] = w
        rel, first = _row_errors(name, x, y, cu)
        rows[name] = (float(rel.max()) if rel.size else 0.0,
                      float(rel[first].max()) if first is not None and first.any() else 0.0)
    gu.log(f"[{label}] worst per-block rel frob: " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    gu.log(f"[{label}] worst row (first tokens of samples): " +
           ", ".join(f"{k} {v[0]:.2e} ({v[1]:.2e})" for k, v in rows.items()))
    for name, w in worst.items():
        assert w <= tol, (label, name, w, tol)
    for name, (w, _) in rows.items():
        assert w <= row_tol, (label, name, "row", w, row_tol)


CASES = [
    ("bf16_d128", (129, 0, 64, 200, 1, 63), 3, 128, 128, "bf16", False, True),
    ("bf16_d128_zero_state", (129, 0, 64, 200, 1, 63), 2, 128, 128, "bf16", False, False),
    ("bf16_d64_128", (70, 33, 0, 100), 2, 64, 128, "bf16", False, True),
    ("bf16_d128_64", (70, 33, 0, 100), 2, 128, 64, "bf16", False, True),
    ("bf16_norm", (129, 0, 64, 200, 1, 63), 2, 128, 128, "bf16", True, True),
    ("f32_d64", (100, 37, 0, 250), 2, 64, 64, "f32", False, True),
    ("f32_d128_norm", (70, 130), 2, 128, 128, "f32", True, True),
    # few long samples: the chains run as two passes over segments of 64 chunks
    # (157, 0, 10 and 66 chunks: three segments, an empty sample, one, two)
    ("bf16_split", (5000, 0, 300, 2100), 2, 128, 128, "bf16", False, True),
    ("f32_split", (2500, 2200), 1, 64, 64, "f32", False, True),
    ("bf16_split_norm_d64_128", (4200,), 1, 64, 128, "bf16", True, True),
    ("bf16_split_zero_state", (4200, 33), 1, 128, 128, "bf16", False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_vs_oracle(case):
    name, lens, H, dk, dv, dt, norm, with_state = case
    spec = inputs.KdaSpec(f"bwd_{name}", lens, H, dk, dv, dt, (0.001, 0.1), 7171)
    gu.log(f"case backward {name}")
    a = inputs.generate(spec)
    if norm:
        a = gu.unnormalised(spec, a, 71)
    do, dfs, s0 = _draw_grads(spec, 72)
    if not with_state:
        dfs = s0 = None
    got = _run(spec, a, do, dfs, s0, norm)
    ref = _oracle(spec, a, do, dfs, s0, norm)
    _compare(spec, got, ref, f"backward {name}")


def test_backward_split_reads_this_calls_transitions():
    """With the chains split into segments, the state-gradient chain's second pass reads the
    transposed segment transitions that the state chain's first pass writes on the other
    stream. Without decay and with a small beta a segment's transition is far from zero (about
    0.85 of the identity over 2,048 tokens), so a transition left in the workspace by an
    earlier call would show in every gradient of the earlier segments: a call on the same
    shapes with the drawn beta (whose transitions have a norm under 0.02) runs first."""
    spec = inputs.KdaSpec("bwd_split_phi", (6000,), 1, 128, 128, "bf16", (0.0, 0.0), 7474)
    gu.log("case backward split: segment transitions of this call (three segments, no decay, small beta)")
    a = inputs.generate(spec)
    do, dfs, s0 = _draw_grads(spec, 75)
    _run(spec, a, do, dfs, s0, False)
    b = dict(a)
    b["beta"] = inputs.f64_to_bf16_bits(0.02 * inputs.to_f64(a["beta"], spec.dtype))
    got = _run(spec, b, do, dfs, s0, False)
    ref = _oracle(spec, b, do, dfs, s0, False)
    _compare(spec, got, ref, "backward split, transitions of this call")


def _sampled(spec, heads, seed):
    """The full-size workload on the GPU (all heads), the oracle on the listed heads (one
    oracle thread per (sample, head))."""
    a = inputs.generate(spec)
    do, _, _ = _draw_grads(spec, seed)
    got = _run(spec, a, do, None, None, False)
    sl = {x: a[x][:, heads] for x in ("q", "k", "v", "log_alpha", "beta")}
    sl["cu_seqlens"] = a["cu_seqlens"]
    sub = inputs.KdaSpec(spec.name, spec.seq_lens, len(heads), spec.dk, spec.dv, spec.dtype,
                         spec.log_alpha_range, spec.seed)
    ref = _oracle(sub, sl, do[:, heads], None, None, False)
    got = [x[:, heads] for x in got]
    _compare(sub, got, ref, f"backward {spec.name} heads {heads}")


def test_backward_config1_all_heads():
    gu.log("case backward config 1 (packed 8 samples, 17,108 tokens), all 16 heads")
    _sampled(inputs.config(1), list(range(16)), 74)


def test_backward_config2_all_heads():
    gu.log("case backward config 2 (4 x 4,352 tokens), all 16 heads")
    _sampled(inputs.config(2), list(range(16)), 75)


def test_backward_config3_all_heads():
    gu.log("case backward config 3 (33,272 tokens, one sample), all 16 heads")
    _sampled(inputs.config(3), list(range(16)), 76)


def test_backward_config4_all_heads():
    """The 30-second-clip workload (one sample of 189,272 tokens, 16 heads, the chains split
    into segments) on the GPU; the oracle on every head (one oracle thread per head, about
    30 s on 16 host threads and 6.5 GB of its checkpoints)."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.config(4)
    heads = list(range(spec.heads))
    gu.log("case backward config 4 (one sample, 189,272 tokens), all 16 heads")
    a = inputs.generate(spec)
    do, _, _ = _draw_grads(spec, 77)
    d = gu.device_inputs(spec, a)
    tdo = torch.from_numpy(do.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    g = kda.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"], tdo)
    torch.cuda.synchronize()
    got = [x[:, heads].float().cpu().double().numpy() for x in g]
    del g, d, tdo
    sl = {x: a[x][:, heads] for x in ("q", "k", "v", "log_alpha", "beta")}
    sl["cu_seqlens"] = a["cu_seqlens"]
    sub = inputs.KdaSpec(spec.name, spec.seq_lens, len(heads), spec.dk, spec.dv, spec.dtype,
                         spec.log_alpha_range, spec.seed)
    ref = _oracle(sub, sl, do[:, heads], None, None, False)
    _compare(sub, got, ref, f"backward {spec.name} heads {heads}")


def test_backward_timing_records_each_kernel():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.KdaSpec("bwd_timing", (300, 77), 2, 128, 128, "bf16", (0.001, 0.1), 7272)
    gu.log("case backward timing")
    a = inputs.generate(spec)
    do, _, _ = _draw_grads(spec, 73)
    kda.timing_enable(True)
    try:
        _run(spec, a, do, None, None, False)
    finally:
        kda.timing_enable(False)
    for name in ("bwd_plan", "bwd_prep", "bwd_state", "bwd_dstate", "bwd_grad"):
        n, ms = kda.timing_read(name)
        assert n == 1 and ms > 0, (name, n, ms)
    torch.cuda.synchronize()


def test_backward_split_timing_records_each_kernel():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.KdaSpec("bwd_split_timing", (4200,), 1, 128, 128, "bf16", (0.001, 0.1), 7373)
    gu.log("case backward split timing")
    a = inputs.generate(spec)
    do, _, _ = _draw_grads(spec, 77)
    kda.timing_enable(True)
    try:
        _run(spec, a, do, None, None, False)
    finally:
        kda.timing_enable(False)
    for name in ("bwd_plan", "bwd_prep", "bwd_state_seg", "bwd_state", "bwd_dstate_seg", "bwd_dstate", "bwd_grad"):
        n, ms = kda.timing_read(name)
        assert n == 1 and ms > 0, (name, n, ms)
    torch.cuda.synchronize()


def test_backward_bitwise_deterministic():
    """Two runs on the same inputs give the same gradients bit for bit (the partial sums of
    dbeta and dgamma are added in a fixed order), also with the chains split."""
    spec = inputs.KdaSpec("bwd_det", (300, 77, 1000, 4200), 1, 128, 128, "bf16", (0.001, 0.1), 7474)
    gu.log("case backward determinism")
    a = inputs.generate(spec)
    do, dfs, s0 = _draw_grads(spec, 78)
    g1 = _run(spec, a, do, dfs, s0, False)
    g2 = _run(spec, a, do, dfs, s0, False)
    for name, x, y in zip(NAMES, g1, g2):
        assert np.array_equal(x, y), name


def test_backward_on_two_caller_streams():
    """The chains run on the caller's stream and a second internal stream, forked after the
    prep and joined before the gradient kernel: two calls enqueued back to back on two other
    streams, with no host synchronisation between them, give the default-stream gradients bit
    for bit."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    spec = inputs.KdaSpec("bwd_streams", (700, 2100, 96), 2, 128, 128, "bf16", (0.001, 0.1), 7475)
    gu.log("case backward on two caller streams")
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    g = torch.Generator(device="cuda:0")
    g.manual_seed(79)
    do = torch.randn((spec.total_tokens, spec.heads, spec.dv), device="cuda:0", generator=g).to(torch.bfloat16)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"], do)
    ref = [t.clone() for t in kda.backward(*args) if t is not None]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        r1 = kda.backward(*args, stream=s1)
    with torch.cuda.stream(s2):
        r2 = kda.backward(*args, stream=s2)
    torch.cuda.synchronize()
    for res in (r1, r2):
        got = [t for t in res if t is not None]
        for x, y in zip(got, ref):
            bx = x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
            by = y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)
            assert torch.equal(bx, by)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_backward_without_decay(dt):
    """log a = 0 (a = 1, no forgetting): every decay factor of the chunked form is exactly 1."""
    spec = inputs.KdaSpec(f"bwd_nodecay_{dt}", (129, 0, 300, 64), 2, 128, 128, dt, (0.0, 0.0), 7272)
    gu.log(f"case backward without decay, {dt}")
    a = inputs.generate(spec)
    do, dfs, s0 = _draw_grads(spec, 73)
    got = _run(spec, a, do, dfs, s0, False)
    ref = _oracle(spec, a, do, dfs, s0, False)
    _compare(spec, got, ref, f"backward without decay {dt}")
