"""GPU parity of kda_short_conv (through the C ABI) against the fp64 oracle.

Bound per element, from the arithmetic: |y - ref| <= u |ref| + 1.01 (n + 1) 2^-24 sum_taps |w| |x|
with u = 2^-8 (one round-to-nearest-even to bf16) for bf16 data and u = 0 for fp32 data; the
second term bounds fp32 accumulation by fused multiply-adds over the n = k_text + k_t*k_h*k_w
taps (the 1.01 covers the bf16 rounding of that error). sum_taps |w||x| is the oracle applied
to |x| and |w| (the operation is linear).
"""
import numpy as np
import pytest

import gpu_util as gu
from delta_rule_recurrent_kda_amd import inputs

pytestmark = pytest.mark.gpu


def _case(seed, shapes, C, ks, dtype):
    """shapes: list of (text_len, T, H, W); ks: (k_text, kt, kh, kw)."""
    rng = np.random.default_rng(seed)
    lens = [L + T * H * W for L, T, H, W in shapes]
    tot = sum(lens)
    x = rng.standard_normal((tot, C))
    x = inputs.bf16_bits_to_f64(inputs.f64_to_bf16_bits(x)) if dtype == "bf16" else x.astype(np.float32).astype(np.float64)
    wt = rng.standard_normal((ks[0], C)).astype(np.float32) * 0.5
    wv = rng.standard_normal((ks[1], ks[2], ks[3], C)).astype(np.float32) * 0.3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tl = np.array([s[0] for s in shapes], np.int32)
    gr = np.array([s[1:] for s in shapes], np.int32).reshape(-1, 3)
    return x, wt, wv, cu, tl, gr


def _run(x, wt, wv, cu, tl, gr, dtype):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    dev = "cuda:0"
    if dtype == "bf16":
        tx = torch.from_numpy(inputs.f64_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        tx = torch.from_numpy(x.astype(np.float32)).to(dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    y = kda.short_conv(tx, t(wt), t(wv), t(cu), t(tl), t(gr))
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def _check(seed, shapes, C, ks, dtype, label):
    import oracle
    x, wt, wv, cu, tl, gr = _case(seed, shapes, C, ks, dtype)
    gu.log(f"case short conv {label}: {len(shapes)} samples, {len(x)} tokens, C={C}, kernels {ks}, {dtype}")
    y = _run(x, wt, wv, cu, tl, gr, dtype)
    ref = oracle.short_conv(x, wt, wv, cu, tl, gr)
    mag = oracle.short_conv(np.abs(x), np.abs(wt), np.abs(wv), cu, tl, gr)
    u = 2.0 ** -8 if dtype == "bf16" else 0.0
    bound = u * np.abs(ref) + 1.01 * (ks[0] + ks[1] * ks[2] * ks[3] + 1) * 2.0 ** -24 * mag
    err = np.abs(y - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    gu.log(f"[{label}] worst error / bound {worst:.3f}, max abs error {err.max(initial=0):.3e}")
    assert np.all(err <= bound), (label, worst)
    assert np.all(y[mag == 0] == 0)


CASES = [
    ("mixed_bf16", [(5, 3, 4, 6), (0, 2, 3, 3), (9, 1, 5, 5), (7, 0, 2, 2), (0, 0, 1, 1), (3, 4, 1, 1)],
     72, (4, 3, 3, 3), "bf16"),
    ("mixed_f32", [(5, 3, 4, 6), (0, 2, 3, 3), (9, 1, 5, 5), (7, 0, 2, 2), (3, 4, 1, 1)], 64, (4, 3, 3, 3), "f32"),
    ("largest_kernels", [(20, 6, 7, 9), (3, 1, 2, 2)], 16, (8, 4, 5, 5), "bf16"),
    ("pointwise", [(6, 2, 3, 3), (0, 1, 4, 4)], 24, (1, 1, 1, 1), "bf16"),
    ("uneven_kernels", [(11, 5, 3, 8)], 8, (2, 2, 3, 1), "f32"),
    ("many_channel_blocks", [(33, 3, 6, 7), (0, 2, 5, 5)], 520, (4, 3, 3, 3), "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_short_conv_vs_oracle(case):
    name, shapes, C, ks, dt = case
    _check(81, shapes, C, ks, dt, name)


def test_short_conv_clip5s_layout():
    # the 5-second clip layout: 512 text tokens + a 21 x 30 x 52 latent grid (33,272 tokens)
    _check(82, [(512, 21, 30, 52)], 128, (4, 3, 3, 3), "bf16", "clip5s layout")


@pytest.mark.parametrize("label,shapes,C,dt", [
    ("clip5s_full_width", [(512, 21, 30, 52)], 2048, "bf16"),   # the benchmark's layout and width
    ("image4", [(256, 1, 64, 64)] * 4, 256, "bf16"),
    ("clip5s_f32", [(512, 21, 30, 52)], 256, "f32"),
])
def test_short_conv_exact_at_full_size(label, shapes, C, dt):
    """Inputs and weights in {-1, 0, 1}: every product and partial sum is exact in fp32 and every
    output (|y| <= 31) exact in bf16, so the kernel must equal the oracle bit for bit."""
    import oracle
    rng = np.random.default_rng(86)
    lens = [L + T * H * W for L, T, H, W in shapes]
    x = rng.integers(-1, 2, (sum(lens), C)).astype(np.float64)
    wt = rng.integers(-1, 2, (4, C)).astype(np.float32)
    wv = rng.integers(-1, 2, (3, 3, 3, C)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tl = np.array([s[0] for s in shapes], np.int32)
    gr = np.array([s[1:] for s in shapes], np.int32).reshape(-1, 3)
    gu.log(f"case short conv exact {label}: {len(x)} tokens, C={C}, {dt}")
    y = _run(x, wt, wv, cu, tl, gr, dt)
    ref = oracle.short_conv(x, wt, wv, cu, tl, gr)
    bad = int(np.count_nonzero(y != ref))
    gu.log(f"[{label}] {bad} of {ref.size} differ")
    assert bad == 0


def test_short_conv_image_batch_layout():
    # four images: 256 text tokens + a 64 x 64 grid each
    _check(83, [(256, 1, 64, 64)] * 4, 64, (4, 3, 3, 3), "bf16", "image4 layout")


def _bound_check(y, ref, mag, label, ntaps=31):
    bound = 2.0 ** -8 * np.abs(ref) + 1.01 * (ntaps + 1) * 2.0 ** -24 * mag
    err = np.abs(y - ref)
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    gu.log(f"[{label}] worst error / bound {worst:.3f}")
    assert np.all(err <= bound), (label, worst)


def test_short_conv_grid_not_matching_length():
    """Samples whose grid does not match their length (the caller's error, not checked unless
    asked): the kernel still reads and writes only inside each sample. Grid positions past a
    sample's last token read as zero, so the present tokens equal the oracle on the full grid
    with the missing tokens zero; tokens past T*H*W equal zero. Packed with a well-formed
    sample, whose output must be unaffected, over 40 channels (a partial channel block)."""
    import oracle
    C, ks = 40, (4, 3, 3, 3)
    # (text_len, grid tokens present, stored grid T, H, W)
    samples = [(4, 47, (3, 4, 5)),      # grid longer than the sample, last frame partial
               (2, 20, (2, 6, 7)),      # first frame partial: rows past the last token
               (3, 10, (1, 3, 50)),     # one row longer than every token present
               (5, 25, (2, 3, 3)),      # grid shorter than the sample: 7 tokens past it
               (6, 9, (0, 3, 3)),       # no frames: every visual token past the grid
               (3, 30, (2, 3, 5))]      # well formed
    rng = np.random.default_rng(85)
    lens = [L + nv for L, nv, _ in samples]
    x = inputs.bf16_bits_to_f64(inputs.f64_to_bf16_bits(rng.standard_normal((sum(lens), C))))
    wt = rng.standard_normal((ks[0], C)).astype(np.float32) * 0.5
    wv = rng.standard_normal((ks[1], ks[2], ks[3], C)).astype(np.float32) * 0.3
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tl = np.array([s[0] for s in samples], np.int32)
    gr = np.array([s[2] for s in samples], np.int32)
    gu.log(f"case short conv grid not matching length: {len(samples)} samples, {len(x)} tokens, C={C}")
    y = _run(x, wt, wv, cu, tl, gr, "bf16")
    for n, (L, nv, (T, H, W)) in enumerate(samples):
        xs = x[cu[n]:cu[n + 1]]
        full = L + T * H * W
        xf = np.zeros((full, C))
        keep = min(L + nv, full)
        xf[:keep] = xs[:keep]
        one = lambda a, u, v: oracle.short_conv(a, u, v, np.array([0, full], np.int32), np.array([L], np.int32),
                                                np.array([[T, H, W]], np.int32))
        ref = np.zeros((L + nv, C))
        mag = np.zeros((L + nv, C))
        ref[:keep] = one(xf, wt, wv)[:keep]
        mag[:keep] = one(np.abs(xf), np.abs(wt), np.abs(wv))[:keep]
        _bound_check(y[cu[n]:cu[n + 1]], ref, mag, f"sample {n} grid {T}x{H}x{W}, {nv} grid tokens")
        assert np.all(y[cu[n] + keep:cu[n + 1]] == 0)


def test_short_conv_timing_hook():
    import torch
    from delta_rule_recurrent_kda_amd import kda
    x, wt, wv, cu, tl, gr = _case(84, [(10, 2, 4, 4)], 32, (4, 3, 3, 3), "bf16")
    kda.timing_enable(True)
    try:
        _run(x, wt, wv, cu, tl, gr, "bf16")
    finally:
        kda.timing_enable(False)
    for name in ("conv_plan", "conv"):
        n, ms = kda.timing_read(name)
        assert n == 1 and ms > 0, name
    torch.cuda.synchronize()
