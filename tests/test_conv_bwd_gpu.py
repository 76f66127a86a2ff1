"""GPU parity of kda_short_conv_backward (through the C ABI) against the fp64 oracle.

Bounds from the arithmetic (u32 = 2^-24, fp32 accumulation with fused multiply-adds):
  dx: |dx - ref| <= u |ref| + 1.01 * (n_taps + 1) * u32 * sum_taps |w| |dy|, u = 2^-8 for bf16
      (one rounding of the fp32 result), 0 for fp32; n_taps = k_text + k_t*k_h*k_w bounds the
      terms of one element.
  dw: |dw - ref| <= (n_terms + 1) * u32 * sum |x| |dy|, n_terms <= the number of tokens, which
      bounds the terms of any order of summation.
sum |w||dy| and sum |x||dy| are the oracle applied to absolute values (the maps are linear).
At full sizes the inputs are small integers, so every product and partial sum is exact in
fp32 (and dx in bf16): there the results must equal the oracle exactly.
"""
import numpy as np
import pytest

import gpu_util as gu
from delta_rule_recurrent_kda_amd import inputs

pytestmark = pytest.mark.gpu


def _tables(shapes):
    lens = [L + T * H * W for L, T, H, W in shapes]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tl = np.array([s[0] for s in shapes], np.int32)
    gr = np.array([s[1:] for s in shapes], np.int32).reshape(-1, 3)
    return cu, tl, gr


def _round(a, dtype):
    return inputs.bf16_bits_to_f64(inputs.f64_to_bf16_bits(a)) if dtype == "bf16" else a.astype(np.float32).astype(np.float64)


def _case(seed, shapes, C, ks, dtype, integer=False):
    rng = np.random.default_rng(seed)
    cu, tl, gr = _tables(shapes)
    tot = int(cu[-1])
    if integer:
        x = rng.integers(-1, 2, (tot, C)).astype(np.float64)
        dy = rng.integers(-1, 2, (tot, C)).astype(np.float64)
        wt = rng.integers(-1, 2, (ks[0], C)).astype(np.float32)
        wv = rng.integers(-1, 2, (ks[1], ks[2], ks[3], C)).astype(np.float32)
    else:
        x = _round(rng.standard_normal((tot, C)), dtype)
        dy = _round(rng.standard_normal((tot, C)), dtype)
        wt = rng.standard_normal((ks[0], C)).astype(np.float32) * 0.5
        wv = rng.standard_normal((ks[1], ks[2], ks[3], C)).astype(np.float32) * 0.3
    return x, dy, wt, wv, cu, tl, gr


def _dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(inputs.f64_to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda:0")


def _run(x, dy, wt, wv, cu, tl, gr, dtype):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    dx, dwt, dwv = kda.short_conv_backward(_dev(x, dtype), t(wt), t(wv), t(cu), t(tl), t(gr), _dev(dy, dtype))
    torch.cuda.synchronize()
    return dx.float().cpu().double().numpy(), dwt.cpu().double().numpy(), dwv.cpu().double().numpy()


def _check(seed, shapes, C, ks, dtype, label):
    import oracle
    x, dy, wt, wv, cu, tl, gr = _case(seed, shapes, C, ks, dtype)
    gu.log(f"case short conv backward {label}: {len(shapes)} samples, {len(x)} tokens, C={C}, kernels {ks}, {dtype}")
    dx, dwt, dwv = _run(x, dy, wt, wv, cu, tl, gr, dtype)
    rdx, rdwt, rdwv = oracle.short_conv_backward(x, wt, wv, cu, tl, gr, dy)
    mdx, mdwt, mdwv = oracle.short_conv_backward(np.abs(x), np.abs(wt), np.abs(wv), cu, tl, gr, np.abs(dy))
    u = 2.0 ** -8 if dtype == "bf16" else 0.0
    ntaps = ks[0] + ks[1] * ks[2] * ks[3]
    bdx = u * np.abs(rdx) + 1.01 * (ntaps + 1) * 2.0 ** -24 * mdx
    e = np.abs(dx - rdx)
    gu.log(f"[{label}] dx worst error / bound {float((e / np.maximum(bdx, 1e-300)).max(initial=0)):.3f}")
    assert np.all(e <= bdx), label
    assert np.all(dx[mdx == 0] == 0)
    n = len(x) + 1
    for name, got, ref, mag in (("dw_text", dwt, rdwt, mdwt), ("dw_vis", dwv, rdwv, mdwv)):
        b = n * 2.0 ** -24 * mag
        e = np.abs(got - ref)
        gu.log(f"[{label}] {name} worst error / bound {float((e / np.maximum(b, 1e-300)).max(initial=0)):.3f}")
        assert np.all(e <= b), (label, name)


CASES = [
    ("mixed_bf16", [(5, 3, 4, 6), (0, 2, 3, 3), (9, 1, 5, 5), (7, 0, 2, 2), (0, 0, 1, 1), (3, 4, 1, 1)],
     72, (4, 3, 3, 3), "bf16"),
    ("mixed_f32", [(5, 3, 4, 6), (0, 2, 3, 3), (9, 1, 5, 5), (7, 0, 2, 2), (3, 4, 1, 1)], 64, (4, 3, 3, 3), "f32"),
    ("largest_kernels", [(20, 6, 7, 9), (3, 1, 2, 2)], 16, (8, 4, 5, 5), "bf16"),
    ("largest_kernels_f32", [(11, 5, 6, 6)], 24, (8, 4, 5, 5), "f32"),
    ("pointwise", [(6, 2, 3, 3), (0, 1, 4, 4)], 24, (1, 1, 1, 1), "bf16"),
    ("uneven_kernels", [(11, 5, 3, 8)], 8, (2, 2, 3, 1), "f32"),
    ("tall_kernel", [(4, 3, 7, 5)], 16, (3, 2, 5, 1), "bf16"),
    ("wide_kernel", [(4, 3, 4, 11)], 16, (3, 2, 1, 5), "bf16"),
    ("many_channel_blocks", [(33, 3, 6, 7), (0, 2, 5, 5)], 520, (4, 3, 3, 3), "bf16"),
    ("many_tiles", [(300, 6, 17, 23), (129, 2, 9, 31)], 64, (4, 3, 3, 3), "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_short_conv_backward_vs_oracle(case):
    name, shapes, C, ks, dt = case
    _check(91, shapes, C, ks, dt, name)


@pytest.mark.parametrize("label,shapes,C,dt", [
    ("clip5s_full_width", [(512, 21, 30, 52)], 2048, "bf16"),   # 5-second clip, 16 heads x 128 channels
    ("image4", [(256, 1, 64, 64)] * 4, 256, "bf16"),            # four images, 256 text tokens + 64 x 64 each
    ("clip5s_f32", [(512, 21, 30, 52)], 256, "f32"),            # the fp32 data path at the clip's layout
])
def test_short_conv_backward_exact_at_full_size(label, shapes, C, dt):
    """Small-integer inputs: every product and partial sum is exact, so the kernels must match
    the oracle bit for bit, at the sizes and launch shape the benchmark uses."""
    import oracle
    ks = (4, 3, 3, 3)
    x, dy, wt, wv, cu, tl, gr = _case(92, shapes, C, ks, dt, integer=True)
    gu.log(f"case short conv backward exact {label}: {len(x)} tokens, C={C}, {dt}")
    dx, dwt, dwv = _run(x, dy, wt, wv, cu, tl, gr, dt)
    rdx, rdwt, rdwv = oracle.short_conv_backward(x, wt, wv, cu, tl, gr, dy)
    for name, got, ref in (("dx", dx, rdx), ("dw_text", dwt, rdwt), ("dw_vis", dwv, rdwv)):
        bad = int(np.count_nonzero(got != ref))
        gu.log(f"[{label}] {name}: {bad} of {ref.size} differ")
        assert bad == 0, (label, name)


def test_short_conv_backward_grid_not_matching_length():
    """Samples whose grid does not match their length: the kernels read and write only inside
    each sample. The expected values are the oracle on the full grid with the missing x and dy
    tokens zero; dx is zero for tokens past T*H*W."""
    import oracle
    C, ks = 40, (4, 3, 3, 3)
    samples = [(4, 47, (3, 4, 5)), (2, 20, (2, 6, 7)), (3, 10, (1, 3, 50)), (5, 25, (2, 3, 3)),
               (6, 9, (0, 3, 3)), (3, 30, (2, 3, 5))]
    rng = np.random.default_rng(93)
    lens = [L + nv for L, nv, _ in samples]
    x = _round(rng.standard_normal((sum(lens), C)), "bf16")
    dy = _round(rng.standard_normal((sum(lens), C)), "bf16")
    wt = rng.standard_normal((ks[0], C)).astype(np.float32) * 0.5
    wv = rng.standard_normal((ks[1], ks[2], ks[3], C)).astype(np.float32) * 0.3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tl = np.array([s[0] for s in samples], np.int32)
    gr = np.array([s[2] for s in samples], np.int32)
    gu.log(f"case short conv backward grid not matching length: {len(samples)} samples, {len(x)} tokens")
    dx, dwt, dwv = _run(x, dy, wt, wv, cu, tl, gr, "bf16")
    rwt = np.zeros_like(dwt)
    rwv = np.zeros_like(dwv)
    mwt = np.zeros_like(dwt)
    mwv = np.zeros_like(dwv)
    for n, (L, nv, (T, H, W)) in enumerate(samples):
        full = L + T * H * W
        keep = min(L + nv, full)
        xf = np.zeros((full, C))
        gf = np.zeros((full, C))
        xf[:keep] = x[cu[n]:cu[n] + keep]
        gf[:keep] = dy[cu[n]:cu[n] + keep]
        tabs = (np.array([0, full], np.int32), np.array([L], np.int32), np.array([[T, H, W]], np.int32))
        rdx, a, b = oracle.short_conv_backward(xf, wt, wv, *tabs, gf)
        mdx, ma, mb = oracle.short_conv_backward(np.abs(xf), np.abs(wt), np.abs(wv), *tabs, np.abs(gf))
        rwt += a
        rwv += b
        mwt += ma
        mwv += mb
        got = dx[cu[n]:cu[n + 1]]
        bound = 2.0 ** -8 * np.abs(rdx[:keep]) + 1.01 * 32 * 2.0 ** -24 * mdx[:keep]
        assert np.all(np.abs(got[:keep] - rdx[:keep]) <= bound), n
        assert np.all(got[keep:] == 0), n
    nb = (len(x) + 1) * 2.0 ** -24
    assert np.all(np.abs(dwt - rwt) <= nb * mwt)
    assert np.all(np.abs(dwv - rwv) <= nb * mwv)


def test_short_conv_backward_no_tokens_gives_zero_weight_gradients():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    dev = "cuda:0"
    C = 16
    for cu_list, tl_list, gr_list in (([0], [], []), ([0, 0, 0], [0, 0], [[0, 1, 1], [0, 3, 3]])):
        N = len(cu_list) - 1
        gu.log(f"case short conv backward no tokens: {N} samples")
        x = torch.zeros((0, C), dtype=torch.bfloat16, device=dev)
        wt = torch.randn((4, C), device=dev)
        wv = torch.randn((3, 3, 3, C), device=dev)
        dwt = torch.full_like(wt, float("nan"))
        dwv = torch.full_like(wv, float("nan"))
        cu = torch.tensor(cu_list, dtype=torch.int32, device=dev)
        tl = torch.tensor(tl_list, dtype=torch.int32, device=dev)
        gr = torch.tensor(gr_list, dtype=torch.int32, device=dev).reshape(-1, 3)
        kda.short_conv_backward(x, wt, wv, cu, tl, gr, x.clone(), torch.empty_like(x), dwt, dwv)
        torch.cuda.synchronize()
        assert torch.all(dwt == 0) and torch.all(dwv == 0)


def test_short_conv_backward_bitwise_deterministic():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    x, dy, wt, wv, cu, tl, gr = _case(94, [(64, 5, 12, 20), (17, 3, 7, 9)], 128, (4, 3, 3, 3), "bf16")
    gu.log(f"case short conv backward determinism: {len(x)} tokens")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    args = (_dev(x, "bf16"), t(wt), t(wv), t(cu), t(tl), t(gr), _dev(dy, "bf16"))
    first = [v.clone() for v in kda.short_conv_backward(*args)]
    for _ in range(3):
        again = kda.short_conv_backward(*args)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_short_conv_backward_timing_hook():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    x, dy, wt, wv, cu, tl, gr = _case(95, [(10, 2, 4, 4)], 32, (4, 3, 3, 3), "bf16")
    kda.timing_enable(True)
    try:
        _run(x, dy, wt, wv, cu, tl, gr, "bf16")
    finally:
        kda.timing_enable(False)
    for name in ("conv_bwd_plan", "conv_dx", "conv_dw", "conv_dw_reduce"):
        n, ms = kda.timing_read(name)
        assert n == 1 and ms > 0, name
    torch.cuda.synchronize()


def test_short_conv_at_the_offset_limit():
    """Tokens x channels just under 2^31, the library's limit for 32-bit element offsets: 21,845
    identical samples (16 text tokens and a 2 x 4 x 4 grid) at 2,048 channels, 4.3 GB per bf16
    tensor. With inputs and weights in {-1, 0, 1} every result is exact, so every sample's y
    and dx must equal the oracle on one sample, and dw_text and dw_vis must equal 21,845 times
    the one-sample weight gradients (|sum| < 2^24)."""
    import torch
    import oracle
    from delta_rule_recurrent_kda_amd import kda
    C, L, grid1 = 2048, 16, (2, 4, 4)
    n1 = L + grid1[0] * grid1[1] * grid1[2]
    N = (2 ** 31 - 1) // (n1 * C)
    assert N * n1 * C < 2 ** 31 and (N + 1) * n1 * C >= 2 ** 31
    ks = (4, 3, 3, 3)
    x1, dy1, wt, wv, cu1, tl1, gr1 = _case(96, [(L, *grid1)], C, ks, "bf16", integer=True)
    y_ref = oracle.short_conv(x1, wt, wv, cu1, tl1, gr1)
    dx_ref, dwt_ref, dwv_ref = oracle.short_conv_backward(x1, wt, wv, cu1, tl1, gr1, dy1)
    gu.log(f"case short conv at the offset limit: {N} samples x {n1} tokens x {C} channels = {N * n1 * C} elements")
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = _dev(x1, "bf16").repeat(N, 1)
    dy = _dev(dy1, "bf16").repeat(N, 1)
    cu = torch.arange(N + 1, dtype=torch.int32, device=dev) * n1
    tl = torch.full((N,), L, dtype=torch.int32, device=dev)
    gr = torch.tensor([list(grid1)], dtype=torch.int32, device=dev).repeat(N, 1)
    y = kda.short_conv(x, t(wt), t(wv), cu, tl, gr)
    torch.cuda.synchronize()
    assert torch.equal(y.view(N, n1, C).float(), t(y_ref).float().unsqueeze(0).expand(N, n1, C))
    del y
    dx, dwt, dwv = kda.short_conv_backward(x, t(wt), t(wv), cu, tl, gr, dy)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(N, n1, C).float(), t(dx_ref).float().unsqueeze(0).expand(N, n1, C))
    assert np.array_equal(dwt.cpu().double().numpy(), N * dwt_ref)
    assert np.array_equal(dwv.cpu().double().numpy(), N * dwv_ref)


def test_short_conv_sample_over_one_gib():
    """One sample of 512 text tokens and a 169 x 30 x 52 grid at 2,048 channels: 1.0006 GiB of
    bf16 grid tokens, past what the kernels address with buffer loads, so they take the checked
    path. Every frame holds the same values (small integers, exact arithmetic), which fixes the
    results from the oracle on the same sample cut to 4 and 5 frames:
      y:  frames 0 and 1 as in the 5-frame sample, every later frame as its frame 2;
      dx: frames up to T-3 as the 5-frame sample's frame 0, the last two as its last two;
      dw: dw(5) + (T - 5) (dw(5) - dw(4)), a frame with every time tap inside the grid adding
          dw(5) - dw(4)."""
    import torch
    import oracle
    from delta_rule_recurrent_kda_amd import kda
    C, L, Tf, Hh, Ww = 2048, 512, 169, 30, 52
    assert Tf * Hh * Ww * C * 2 > 1 << 30
    ks = (4, 3, 3, 3)
    rng = np.random.default_rng(97)
    xt = rng.integers(-1, 2, (L, C)).astype(np.float64)
    gt = rng.integers(-1, 2, (L, C)).astype(np.float64)
    xf = rng.integers(-1, 2, (Hh * Ww, C)).astype(np.float64)      # one frame, repeated
    gf = rng.integers(-1, 2, (Hh * Ww, C)).astype(np.float64)
    wt = rng.integers(-1, 2, (ks[0], C)).astype(np.float32)
    wv = rng.integers(-1, 2, (ks[1], ks[2], ks[3], C)).astype(np.float32)

    def ref(nf):
        x = np.concatenate([xt] + [xf] * nf)
        g = np.concatenate([gt] + [gf] * nf)
        tabs = (np.array([0, len(x)], np.int32), np.array([L], np.int32), np.array([[nf, Hh, Ww]], np.int32))
        return oracle.short_conv(x, wt, wv, *tabs), oracle.short_conv_backward(x, wt, wv, *tabs, g)

    y5, (dx5, dwt5, dwv5) = ref(5)
    _, (_, dwt4, dwv4) = ref(4)
    gu.log(f"case short conv sample over 1 GiB: {L + Tf * Hh * Ww} tokens, C={C}")
    dev = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    fr = Hh * Ww
    x = torch.cat([_dev(xt, "bf16"), _dev(xf, "bf16").repeat(Tf, 1)])
    dy = torch.cat([_dev(gt, "bf16"), _dev(gf, "bf16").repeat(Tf, 1)])
    tabs = (t(np.array([0, len(x)], np.int32)), t(np.array([L], np.int32)), t(np.array([[Tf, Hh, Ww]], np.int32)))
    y = kda.short_conv(x, t(wt), t(wv), *tabs).float()
    torch.cuda.synchronize()
    y5t = t(y5).float()
    assert torch.equal(y[:L + 2 * fr], y5t[:L + 2 * fr])
    assert torch.equal(y[L + 2 * fr:].view(Tf - 2, fr, C), y5t[L + 2 * fr:L + 3 * fr].unsqueeze(0).expand(Tf - 2, fr, C))
    del y
    dx, dwt, dwv = kda.short_conv_backward(x, t(wt), t(wv), *tabs, dy)
    torch.cuda.synchronize()
    dx = dx.float()
    dx5t = t(dx5).float()
    assert torch.equal(dx[:L], dx5t[:L])
    assert torch.equal(dx[L:L + (Tf - 2) * fr].view(Tf - 2, fr, C),
                       dx5t[L:L + fr].unsqueeze(0).expand(Tf - 2, fr, C))
    assert torch.equal(dx[L + (Tf - 2) * fr:], dx5t[L + 3 * fr:])
    assert np.array_equal(dwt.cpu().double().numpy(), dwt5 + (Tf - 5) * (dwt5 - dwt4))
    assert np.array_equal(dwv.cpu().double().numpy(), dwv5 + (Tf - 5) * (dwv5 - dwv4))
