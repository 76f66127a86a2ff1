"""Checks that pin the fp64 reverse mode of the short convolution to facts outside it.

Each check takes the pinned forward oracle ``conv(x, w_text, w_vis, cu, text_len, grid) -> y``
and the reverse mode ``conv_bwd(x, w_text, w_vis, cu, text_len, grid, dy) -> (dx, dw_text,
dw_vis)``, and raises AssertionError on a mismatch. The convolution (Chimera, arXiv
2607.28611, paper Sec. 3.4) is linear in x and, separately, in the weights, so its
gradients are the transposes of those two linear maps.
"""
import numpy as np


def _problem(rng, shapes, C, ks):
    lens = [L + T * H * W for L, T, H, W in shapes]
    x = rng.standard_normal((sum(lens), C))
    wt = rng.standard_normal((ks[0], C))
    wv = rng.standard_normal((ks[1], ks[2], ks[3], C))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tl = np.array([s[0] for s in shapes], np.int32)
    gr = np.array([s[1:] for s in shapes], np.int32).reshape(-1, 3)
    return x, wt, wv, cu, tl, gr


def pin_conv_bwd_adjoint(conv, conv_bwd, seed=50):
    """<y, dy> = <x, dx> = <w_text, dw_text> + <w_vis, dw_vis> (linearity in x and in w),
    over a pack with a text-only sample, a grid-only sample, an empty one and a mixed one."""
    rng = np.random.default_rng(seed)
    shapes = [(6, 0, 1, 1), (0, 3, 4, 5), (0, 0, 1, 1), (5, 2, 3, 7)]
    x, wt, wv, cu, tl, gr = _problem(rng, shapes, 3, (4, 3, 3, 5))
    dy = rng.standard_normal(x.shape)
    y = conv(x, wt, wv, cu, tl, gr)
    dx, dwt, dwv = conv_bwd(x, wt, wv, cu, tl, gr, dy)
    lhs = float(np.sum(y * dy))
    sx = float(np.sum(x * dx))
    sw = float(np.sum(wt * dwt) + np.sum(wv * dwv))
    scale = float(np.sum(np.abs(y) * np.abs(dy))) + 1e-300
    assert abs(lhs - sx) <= 1e-12 * scale, (lhs, sx)
    assert abs(lhs - sw) <= 1e-12 * scale, (lhs, sw)


def pin_conv_bwd_dense(conv, conv_bwd, seed=51):
    """Brute force on a tiny pack: the matrices of x -> y and w -> y built column by column
    from unit inputs through the forward; dx and dw are their transposes applied to dy."""
    rng = np.random.default_rng(seed)
    shapes = [(3, 2, 2, 3), (2, 0, 1, 1)]
    ks = (2, 2, 3, 3)
    x, wt, wv, cu, tl, gr = _problem(rng, shapes, 2, ks)
    T, C = x.shape
    dy = rng.standard_normal(x.shape)
    dx, dwt, dwv = conv_bwd(x, wt, wv, cu, tl, gr, dy)
    # x -> y: depthwise, so one unit token in every channel gives the columns of all channels
    A = np.zeros((C, T, T))
    for s in range(T):
        e = np.zeros((T, C))
        e[s] = 1.0
        A[:, :, s] = conv(e, wt, wv, cu, tl, gr).T
    ref_dx = np.stack([A[c].T @ dy[:, c] for c in range(C)], axis=1)
    assert np.allclose(dx, ref_dx, rtol=1e-12, atol=1e-12)
    # w -> y: one unit tap in every channel
    nt = ks[0] + ks[1] * ks[2] * ks[3]
    B = np.zeros((C, T, nt))
    for tap in range(nt):
        ut = np.zeros_like(wt)
        uv = np.zeros_like(wv)
        if tap < ks[0]:
            ut[tap] = 1.0
        else:
            uv.reshape(-1, C)[tap - ks[0]] = 1.0
        B[:, :, tap] = conv(x, ut, uv, cu, tl, gr).T
    ref_dw = np.stack([B[c].T @ dy[:, c] for c in range(C)], axis=1)
    assert np.allclose(dwt, ref_dw[:ks[0]], rtol=1e-12, atol=1e-12)
    assert np.allclose(dwv.reshape(-1, C), ref_dw[ks[0]:], rtol=1e-12, atol=1e-12)


def pin_conv_bwd_modalities_apart(conv, conv_bwd, seed=52):
    """A gradient on the text outputs reaches only text inputs and text taps; one on the grid
    outputs only grid inputs and visual taps; no sample's gradient reaches another."""
    rng = np.random.default_rng(seed)
    shapes = [(5, 2, 3, 4), (4, 1, 2, 2)]
    x, wt, wv, cu, tl, gr = _problem(rng, shapes, 2, (3, 2, 3, 3))
    text = np.zeros(len(x), bool)
    for n in range(2):
        text[cu[n]:cu[n] + tl[n]] = True
    dy_t = rng.standard_normal(x.shape) * text[:, None]
    dx, dwt, dwv = conv_bwd(x, wt, wv, cu, tl, gr, dy_t)
    assert np.all(dx[~text] == 0) and np.all(dwv == 0)
    dy_v = rng.standard_normal(x.shape) * (~text)[:, None]
    dx, dwt, dwv = conv_bwd(x, wt, wv, cu, tl, gr, dy_v)
    assert np.all(dx[text] == 0) and np.all(dwt == 0)
    dy_0 = rng.standard_normal(x.shape)
    dy_0[cu[1]:] = 0.0
    dx, _, _ = conv_bwd(x, wt, wv, cu, tl, gr, dy_0)
    assert np.all(dx[cu[1]:] == 0)


ALL_CONV_BWD_PINS = [pin_conv_bwd_adjoint, pin_conv_bwd_dense, pin_conv_bwd_modalities_apart]
