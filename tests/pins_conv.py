"""Checks that pin the fp64 short-convolution oracle to facts outside it.

Each check takes ``conv(x, w_text, w_vis, cu_seqlens, text_len, grid) -> y`` and raises
AssertionError on a mismatch. The operation (Chimera, arXiv 2607.28611, paper Sec. 3.4 and
the NoPE discussion of position selection; explainer page "What RoPE was actually doing"):
a depthwise kernel per channel; text tokens mixed causally along the token index, visual
tokens mixed over the (T, H, W) grid, causally in time, centred in space; modalities and
samples never read each other.
"""
import numpy as np


def _sample(rng, L, T, H, W, C):
    return rng.standard_normal((L + T * H * W, C))


def _pack(parts):
    x = np.concatenate([p[0] for p in parts])
    cu = np.concatenate([[0], np.cumsum([len(p[0]) for p in parts])]).astype(np.int32)
    tl = np.array([p[1] for p in parts], np.int32)
    gr = np.array([p[2] for p in parts], np.int32).reshape(-1, 3)
    return x, cu, tl, gr


def pin_conv_text_textbook(conv, seed=40):
    """All-text sample: each channel is the textbook causal convolution (np.convolve, full,
    truncated to the sample)."""
    rng = np.random.default_rng(seed)
    L, C, kx = 23, 6, 4
    x = rng.standard_normal((L, C))
    wt = rng.standard_normal((kx, C))
    y = conv(x, wt, rng.standard_normal((2, 3, 3, C)), [0, L], [L], [[0, 2, 2]])
    for c in range(C):
        ref = np.convolve(x[:, c], wt[:, c])[:L]
        assert np.allclose(y[:, c], ref, rtol=1e-12, atol=1e-12), c


def pin_conv_visual_library(conv, seed=41):
    """Grid-only sample: each channel equals scipy.signal.correlate on the grid padded with
    kt-1 zero frames in front and (k-1)/2 zeros on each side in space, the kernel reversed in
    time, 'valid' mode."""
    from scipy import signal
    rng = np.random.default_rng(seed)
    T, H, W, C = 5, 4, 6, 3
    kt, kh, kw = 3, 3, 5
    x = _sample(rng, 0, T, H, W, C)
    wv = rng.standard_normal((kt, kh, kw, C))
    y = conv(x, rng.standard_normal((2, C)), wv, [0, len(x)], [0], [[T, H, W]])
    for c in range(C):
        g = x[:, c].reshape(T, H, W)
        xp = np.pad(g, ((kt - 1, 0), ((kh - 1) // 2,) * 2, ((kw - 1) // 2,) * 2))
        ref = signal.correlate(xp, wv[::-1, :, :, c], mode="valid")
        assert ref.shape == (T, H, W)
        assert np.allclose(y[:, c].reshape(T, H, W), ref, rtol=1e-12, atol=1e-12), c


def pin_conv_shifts(conv, seed=42):
    """A kernel with a single 1 is a shift with zero fill, per modality."""
    rng = np.random.default_rng(seed)
    L, T, H, W, C = 7, 3, 4, 5, 2
    kx, kt, kh, kw = 3, 2, 3, 3
    x = _sample(rng, L, T, H, W, C)
    cu, tl, gr = [0, len(x)], [L], [[T, H, W]]
    for i in range(kx):
        wt = np.zeros((kx, C)); wt[i] = 1.0
        y = conv(x, wt, np.zeros((kt, kh, kw, C)), cu, tl, gr)
        ref = np.zeros((L, C)); ref[i:] = x[:L - i]
        assert np.array_equal(y[:L], ref) and np.all(y[L:] == 0), ("text", i)
    g = x[L:].reshape(T, H, W, C)
    for a in range(kt):
        for b in range(kh):
            for d in range(kw):
                wv = np.zeros((kt, kh, kw, C)); wv[a, b, d] = 1.0
                y = conv(x, np.zeros((kx, C)), wv, cu, tl, gr)
                ref = np.zeros_like(g)
                db, dd = b - (kh - 1) // 2, d - (kw - 1) // 2
                for i in range(T):
                    for j in range(H):
                        for k in range(W):
                            ii, jj, kk = i - a, j + db, k + dd
                            if 0 <= ii and 0 <= jj < H and 0 <= kk < W:
                                ref[i, j, k] = g[ii, jj, kk]
                assert np.array_equal(y[L:].reshape(T, H, W, C), ref) and np.all(y[:L] == 0), (a, b, d)


def pin_conv_separation_causality_packing(conv, seed=43):
    """Text and visual outputs do not depend on the other modality; frame i does not depend
    on later frames; packing and pack order change nothing, bit for bit."""
    rng = np.random.default_rng(seed)
    C = 3
    wt = rng.standard_normal((4, C))
    wv = rng.standard_normal((3, 3, 3, C))
    shapes = [(5, 3, 2, 4), (0, 2, 3, 3), (9, 1, 4, 4), (4, 0, 3, 3)]
    parts = [(_sample(rng, L, T, H, W, C), L, (T, H, W)) for L, T, H, W in shapes]
    x, cu, tl, gr = _pack(parts)
    y = conv(x, wt, wv, cu, tl, gr)
    # each sample alone, and the pack reversed
    for n, (xs, L, g) in enumerate(parts):
        ys = conv(xs, wt, wv, [0, len(xs)], [L], [g])
        assert np.array_equal(ys, y[cu[n]:cu[n + 1]]), n
    xr, cur, tlr, grr = _pack(parts[::-1])
    yr = conv(xr, wt, wv, cur, tlr, grr)
    for n in range(len(parts)):
        m = len(parts) - 1 - n
        assert np.array_equal(yr[cur[m]:cur[m + 1]], y[cu[n]:cu[n + 1]])
    # modality separation and causality in time on sample 0 (5 text tokens, 3 frames of 2x4)
    L, (T, H, W) = 5, (3, 2, 4)
    x2 = x.copy(); x2[cu[0]:cu[0] + L] += 1.0                 # change the text
    y2 = conv(x2, wt, wv, cu, tl, gr)
    assert np.array_equal(y2[cu[0] + L:], y[cu[0] + L:])
    x3 = x.copy(); x3[cu[0] + L:cu[1]] += 1.0                 # change the grid
    y3 = conv(x3, wt, wv, cu, tl, gr)
    assert np.array_equal(y3[:cu[0] + L], y[:cu[0] + L]) and np.array_equal(y3[cu[1]:], y[cu[1]:])
    x4 = x.copy(); x4[cu[0] + L + 2 * H * W:cu[1]] += 1.0     # change the last frame
    y4 = conv(x4, wt, wv, cu, tl, gr)
    assert np.array_equal(y4[:cu[0] + L + 2 * H * W], y[:cu[0] + L + 2 * H * W])
    assert not np.array_equal(y4[cu[0] + L + 2 * H * W:cu[1]], y[cu[0] + L + 2 * H * W:cu[1]])


def pin_conv_image_and_linearity(conv, seed=44):
    """A one-frame grid (an image) ignores the taps on earlier frames; the output is linear
    in the weights."""
    rng = np.random.default_rng(seed)
    C = 4
    x = _sample(rng, 3, 1, 5, 6, C)
    args = ([0, len(x)], [3], [[1, 5, 6]])
    wt = rng.standard_normal((2, C))
    wv = rng.standard_normal((3, 3, 3, C))
    y = conv(x, wt, wv, *args)
    wv2 = wv.copy(); wv2[1:] = rng.standard_normal(wv2[1:].shape)
    assert np.array_equal(conv(x, wt, wv2, *args), y)
    wt3, wv3 = rng.standard_normal(wt.shape), rng.standard_normal(wv.shape)
    ysum = conv(x, wt + wt3, wv + wv3, *args)
    assert np.allclose(ysum, y + conv(x, wt3, wv3, *args), rtol=1e-12, atol=1e-12)


ALL_CONV_PINS = [pin_conv_text_textbook, pin_conv_visual_library, pin_conv_shifts,
                 pin_conv_separation_causality_packing, pin_conv_image_and_linearity]
