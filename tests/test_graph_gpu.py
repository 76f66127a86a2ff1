"""Calls captured in a HIP graph (torch.cuda.CUDAGraph over the library's launches on the
capture stream) replay to the same results as eager calls, bit for bit, with new inputs
copied into the captured buffers between replays (GPU).

The library's workspaces are stream-ordered allocations and the backward forks and joins an
auxiliary stream by events, all of which capture; no call records a memset.
"""
import numpy as np
import pytest

import gpu_util as gu
from delta_rule_recurrent_kda_amd import inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _replays(fn, outs, refill, label, reps=3):
    """Capture fn, then for each replay: refill inputs eagerly, replay, and compare with an
    eager call on the same inputs."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                    # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for rep in range(1, reps + 1):
        refill(rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        fn()
        torch.cuda.synchronize()
        for a, b in zip(got, outs):
            assert torch.equal(_bits(a), _bits(b)), (label, rep)
    gu.log(f"[{label}] {reps} replays equal eager calls")


def test_scan_forward_and_backward_in_a_graph():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    lens = [700, 129, 1500, 0, 37]
    specs = [inputs.custom(lens, heads=4, d=128, seed=21 + s) for s in range(4)]
    drafts = [gu.device_inputs(sp, inputs.generate(sp)) for sp in specs]
    spec = specs[0]
    gu.log("case scan in a graph")
    st = {k: v.clone() for k, v in drafts[0].items()}
    N, T = len(lens), spec.total_tokens
    out = torch.empty((T, spec.heads, spec.dv), dtype=torch.bfloat16, device="cuda:0")
    fs = torch.empty((N, spec.heads, spec.dk, spec.dv), dtype=torch.float32, device="cuda:0")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(22)
    do = torch.randn((T, spec.heads, spec.dv), device="cuda:0", generator=g).to(torch.bfloat16)
    grads = [torch.empty_like(st[n]) for n in ("q", "k", "v", "log_alpha", "beta")]
    dinit = torch.empty_like(fs)

    def refill(rep):
        for k in st:
            st[k].copy_(drafts[rep][k])

    def fwd():
        kda.kda_forward(st["q"], st["k"], st["v"], st["log_alpha"], st["beta"], st["cu_seqlens"], out, fs)

    def bwd():
        r = kda.kda_backward_raw(*[kda._ptr(st[n]) for n in ("q", "k", "v", "log_alpha", "beta", "cu_seqlens")],
                                 None, kda._ptr(do), None, *[kda._ptr(x) for x in grads], kda._ptr(dinit), T, N,
                                 spec.heads, spec.dk, spec.dv, kda.KDA_BF16, 0,
                                 torch.cuda.current_stream().cuda_stream)
        assert r == 0, kda.library().kda_last_error()

    _replays(fwd, [out, fs], refill, "forward")
    _replays(bwd, grads + [dinit], refill, "backward")


def test_short_conv_and_backward_in_a_graph():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    rng = np.random.default_rng(23)
    shapes = [(40, 3, 6, 7), (0, 2, 5, 5), (17, 0, 1, 1)]
    C = 128
    lens = [L + T * H * W for L, T, H, W in shapes]
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    xs = [torch.randn((sum(lens), C), device=dev).to(torch.bfloat16) for _ in range(4)]
    dys = [torch.randn((sum(lens), C), device=dev).to(torch.bfloat16) for _ in range(4)]
    x, dy = xs[0].clone(), dys[0].clone()
    wt = t(rng.standard_normal((4, C)).astype(np.float32))
    wv = t(rng.standard_normal((3, 3, 3, C)).astype(np.float32))
    cu = t(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
    tl = t(np.array([s[0] for s in shapes], np.int32))
    gr = t(np.array([s[1:] for s in shapes], np.int32))
    y, dx, dwt, dwv = torch.empty_like(x), torch.empty_like(x), torch.empty_like(wt), torch.empty_like(wv)
    gu.log("case short convolution in a graph")

    def refill(rep):
        x.copy_(xs[rep])
        dy.copy_(dys[rep])

    _replays(lambda: kda.short_conv(x, wt, wv, cu, tl, gr, y), [y], refill, "short conv")
    _replays(lambda: kda.short_conv_backward(x, wt, wv, cu, tl, gr, dy, dx, dwt, dwv), [dx, dwt, dwv], refill,
             "short conv backward")
