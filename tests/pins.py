"""Checks that pin the fp64 oracle to facts outside itself.

Each check takes ``fwd(q, k, v, log_alpha, beta, cu_seqlens) -> (out, final_state)``
(fp64 arrays, shapes [T, H, d], [T, H], [N+1]) and raises AssertionError on a
mismatch. They hold for the KDA scan of Chimera (arXiv 2607.28611): update
S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T (explainer
page, "One stream, three mechanisms, no positions"), reset S_0 = 0 at packed
sample boundaries and S_t = post-update state (paper Sec. 3, KDA paragraph),
half-life n = ln 0.5 / ln alpha (explainer, same section), readout o_t = S_t^T q_t.
"""
import json
import os

import numpy as np

import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_case(rng, lens, H, dk, dv, unit_keys=True, la_range=(0.01, 0.3)):
    T = int(sum(lens))
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=2, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -rng.uniform(*la_range, (T, H, dk))
    b = rng.uniform(0.0, 1.0, (T, H))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, la, b, cu


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# -- P0: hand-derived worked example (tests/golden/worked_example.json) -------
def pin_worked_example(fwd):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    k = np.array(g["k"], float)[:, None, :]
    v = np.array(g["v"], float)[:, None, :]
    q = np.array(g["q"], float)[:, None, :]
    la = np.log(np.array(g["alpha"], float))[:, None, :]
    b = np.array(g["beta"], float)[:, None]
    cu = np.array(g["cu_seqlens"], np.int32)
    out, fs = fwd(q, k, v, la, b, cu)
    assert np.allclose(out[:, 0], np.array(g["out"]), rtol=0, atol=1e-13), out[:, 0]
    assert np.allclose(fs[:, 0], np.array(g["final_state"]), rtol=0, atol=1e-13), fs[:, 0]


# -- P1: brute force with dense transition matrices -----------------------------
def pin_brute_force(fwd, seed=0):
    rng = np.random.default_rng(seed)
    for lens, H, dk, dv, unit in [((7, 0, 13, 20), 2, 5, 3, True), ((40,), 1, 8, 8, False),
                                  ((1, 2, 3), 3, 3, 6, True)]:
        q, k, v, la, b, cu = _rand_case(rng, lens, H, dk, dv, unit_keys=unit)
        out, fs = fwd(q, k, v, la, b, cu)
        ob, fb = brute.scan_matrices(q, k, v, la, b, cu)
        assert _rel(out, ob) < 1e-12, _rel(out, ob)
        assert _rel(fs, fb) < 1e-12, _rel(fs, fb)
        for n in range(len(lens)):
            for h in range(H):
                fu = brute.final_state_unrolled(k, v, la, b, cu[n], cu[n + 1], h)
                assert np.allclose(fs[n, h], fu, rtol=1e-11, atol=1e-12)


# -- P2: beta = 0 never writes: S and o are exactly zero ------------------------
def pin_beta_zero(fwd, seed=1):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (9, 17), 2, 6, 4)
    b[:] = 0.0
    out, fs = fwd(q, k, v, la, b, cu)
    assert np.all(out == 0.0) and np.all(fs == 0.0)


# -- P3: exact recall with alpha = 1, beta = 1 and orthonormal keys -------------
def pin_exact_recall(fwd, seed=2):
    rng = np.random.default_rng(seed)
    d = 8
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T                                   # orthonormal rows
    T = d + 3
    k = np.zeros((T, 1, d)); v = rng.standard_normal((T, 1, d)); q = np.zeros((T, 1, d))
    for t in range(d):
        k[t, 0] = keys[t]
    # re-write keys 2, 5, 2 with new values: the latest write must win
    for t, s in zip(range(d, T), (2, 5, 2)):
        k[t, 0] = keys[s]
    la = np.zeros((T, 1, d)); b = np.ones((T, 1))
    # query at t asks for the key written at s(t) <= t
    src = [0, 0, 1, 3, 2, 4, 5, 1, 0, 5, 2]
    for t in range(T):
        q[t, 0] = keys[src[t]] if src[t] < d else 0
    cu = np.array([0, T], np.int32)
    out, _ = fwd(q, k, v, la, b, cu)
    for t in range(T):
        s = src[t]
        last = max(u for u in range(t + 1) if np.allclose(k[u, 0], keys[s]))
        assert np.allclose(out[t, 0], v[last, 0], rtol=0, atol=1e-12), (t, s, last)
    # the readout at a write step returns the value just written (post-update state)
    q2 = k.copy()
    out2, _ = fwd(q2, k, v, la, b, cu)
    assert np.allclose(out2[:, 0], v[:, 0], rtol=0, atol=1e-12)


# -- P4: decay-only half-life n = ln 0.5 / ln alpha per key channel -------------
def pin_half_life(fwd):
    d = 4
    n_half = np.array([1, 3, 7, 20])
    alpha = 0.5 ** (1.0 / n_half)
    assert np.allclose(np.log(0.5) / np.log(alpha), n_half)
    T = 1 + 2 * int(n_half.max())
    dv = 3
    k = np.zeros((T, 1, d)); k[0, 0] = np.ones(d) / 2.0       # unit key touching every channel
    v = np.zeros((T, 1, dv)); v[0, 0] = [1.0, -2.0, 0.5]
    b = np.zeros((T, 1)); b[0, 0] = 1.0
    la = np.tile(np.log(alpha), (T, 1))[:, None, :]
    cu = np.array([0, T], np.int32)
    for c in range(d):
        q = np.zeros((T, 1, d)); q[:, 0, c] = 1.0               # reads row c of S
        out, _ = fwd(q, k, v, la, b, cu)
        row0 = out[0, 0]
        assert np.allclose(row0, 0.5 * v[0, 0], atol=1e-14)
        n = int(n_half[c])
        assert np.allclose(out[n, 0], 0.5 * row0, rtol=1e-12, atol=1e-15), (c, out[n, 0], row0)
        assert np.allclose(out[2 * n, 0], 0.25 * row0, rtol=1e-12, atol=1e-15)


# -- P5: reset at boundaries; packing order and packing itself change nothing ---
def pin_reset_and_packing(fwd, seed=3):
    rng = np.random.default_rng(seed)
    lens = [11, 5, 23]
    q, k, v, la, b, cu = _rand_case(rng, lens, 2, 6, 5)
    out, fs = fwd(q, k, v, la, b, cu)
    segs = [slice(cu[i], cu[i + 1]) for i in range(3)]
    order = [2, 0, 1]
    cat = lambda a: np.concatenate([a[segs[i]] for i in order])
    cu2 = np.concatenate([[0], np.cumsum([lens[i] for i in order])]).astype(np.int32)
    out2, fs2 = fwd(cat(q), cat(k), cat(v), cat(la), cat(b), cu2)
    for j, i in enumerate(order):
        assert np.array_equal(out2[cu2[j]:cu2[j + 1]], out[segs[i]])
        assert np.array_equal(fs2[j], fs[i])
    for i in range(3):
        one = np.array([0, lens[i]], np.int32)
        o1, f1 = fwd(q[segs[i]], k[segs[i]], v[segs[i]], la[segs[i]], b[segs[i]], one)
        assert np.array_equal(o1, out[segs[i]]) and np.array_equal(f1[0], fs[i])
    # a zero-length sample yields a zero final state and shifts nothing
    cu3 = np.array([0, lens[0], lens[0], lens[0] + lens[1], sum(lens)], np.int32)
    o3, f3 = fwd(q, k, v, la, b, cu3)
    assert np.array_equal(o3, out) and np.all(f3[1] == 0)
    assert np.array_equal(f3[[0, 2, 3]], fs)


# -- P6: write-readback identity for unit keys -----------------------------------
def pin_write_readback(fwd, seed=4):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (30,), 1, 6, 4)
    for t in (1, 9, 29):
        cu_p = np.array([0, t], np.int32)
        _, fprev = fwd(q[:t], k[:t], v[:t], la[:t], b[:t], cu_p)
        q2 = q[:t + 1].copy(); q2[t] = k[t]
        out, _ = fwd(q2, k[:t + 1], v[:t + 1], la[:t + 1], b[:t + 1], np.array([0, t + 1], np.int32))
        Sd = np.exp(la[t, 0])[:, None] * fprev[0, 0]
        want = (1 - b[t, 0]) * (Sd.T @ k[t, 0]) + b[t, 0] * v[t, 0]
        assert np.allclose(out[t, 0], want, rtol=1e-12, atol=1e-13)


# -- P7: value columns are separable ----------------------------------------------
def pin_column_separability(fwd, seed=5):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (12, 19), 2, 5, 6)
    out, fs = fwd(q, k, v, la, b, cu)
    perm = rng.permutation(6)
    out2, fs2 = fwd(q, k, v[:, :, perm], la, b, cu)
    assert np.allclose(out2, out[:, :, perm], rtol=1e-13, atol=1e-14)
    assert np.allclose(fs2, fs[..., perm], rtol=1e-13, atol=1e-14)
    v3 = v.copy(); v3[:, :, 2] = 0
    out3, fs3 = fwd(q, k, v3, la, b, cu)
    assert np.all(out3[:, :, 2] == 0) and np.all(fs3[..., 2] == 0)


# -- P8: linear in V and in Q when S_0 = 0 ------------------------------------------
def pin_linearity(fwd, seed=6):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (25,), 1, 6, 4)
    v2 = rng.standard_normal(v.shape); q2 = rng.standard_normal(q.shape)
    a1, a2 = 0.7, -1.3
    o1, f1 = fwd(q, k, v, la, b, cu)
    o2, f2 = fwd(q, k, v2, la, b, cu)
    o12, f12 = fwd(q, k, a1 * v + a2 * v2, la, b, cu)
    assert np.allclose(o12, a1 * o1 + a2 * o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(f12, a1 * f1 + a2 * f2, rtol=1e-12, atol=1e-12)
    oq, _ = fwd(q2, k, v, la, b, cu)
    oqq, _ = fwd(a1 * q + a2 * q2, k, v, la, b, cu)
    assert np.allclose(oqq, a1 * o1 + a2 * oq, rtol=1e-12, atol=1e-12)


# -- P9: permuting key channels of q, k, log alpha permutes the state rows only ------
def pin_channel_equivariance(fwd, seed=7):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (21,), 2, 7, 3)
    out, fs = fwd(q, k, v, la, b, cu)
    p = rng.permutation(7)
    out2, fs2 = fwd(q[..., p], k[..., p], v, la[..., p], b, cu)
    assert np.allclose(out2, out, rtol=1e-12, atol=1e-13)
    assert np.allclose(fs2, fs[:, :, p, :], rtol=1e-12, atol=1e-13)


# -- P10: d_k = d_v = 1 is the first-order linear recurrence ------------------------
def pin_scalar_closed_form(fwd, seed=8):
    rng = np.random.default_rng(seed)
    T = 40
    k = rng.uniform(-1.2, 1.2, (T, 1, 1)); v = rng.standard_normal((T, 1, 1))
    q = rng.standard_normal((T, 1, 1)); la = -rng.uniform(0, 0.5, (T, 1, 1))
    b = rng.uniform(0, 1, (T, 1))
    out, fs = fwd(q, k, v, la, b, np.array([0, T], np.int32))
    a = np.exp(la[:, 0, 0]) * (1 - b[:, 0] * k[:, 0, 0] ** 2)     # s_t = a_t s_{t-1} + c_t
    c = b[:, 0] * k[:, 0, 0] * v[:, 0, 0]
    s = np.array([sum(np.prod(a[r + 1:t + 1]) * c[r] for r in range(t + 1)) for t in range(T)])
    assert np.allclose(out[:, 0, 0], s * q[:, 0, 0], rtol=1e-11, atol=1e-13)
    assert np.isclose(fs[0, 0, 0, 0], s[-1], rtol=1e-11, atol=1e-13)


# -- P11: with alpha = 1 a step is one LMS (Widrow-Hoff) step on ||S^T k - v||^2/2 ----
def pin_lms_step(fwd, seed=9):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (15,), 1, 5, 4, unit_keys=False)
    la[:] = 0.0
    _, f14 = fwd(q[:14], k[:14], v[:14], la[:14], b[:14], np.array([0, 14], np.int32))
    _, f15 = fwd(q, k, v, la, b, cu)
    S, kt, vt, bt = f14[0, 0], k[14, 0], v[14, 0], b[14, 0]
    grad = np.outer(kt, S.T @ kt - vt)                  # gradient of 0.5 ||S^T k - v||^2
    assert np.allclose(f15[0, 0], S - bt * grad, rtol=1e-12, atol=1e-13)


# -- P12: contraction: ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t|| for unit keys ------
def pin_contraction(fwd, seed=10):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (60,), 1, 6, 5)
    prev = 0.0
    for t in range(1, 61):
        _, f = fwd(q[:t], k[:t], v[:t], la[:t], b[:t], np.array([0, t], np.int32))
        nrm = np.linalg.norm(f[0, 0], 2)
        assert nrm <= prev + b[t - 1, 0] * np.linalg.norm(v[t - 1, 0]) + 1e-12
        prev = nrm


# -- NaN stays inside its own (sample, head) unit -------------------------------------
def pin_nan_confined(fwd, seed=11):
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, (8, 8, 8), 2, 4, 4)
    v[10, 1, 2] = np.nan                                # sample 1, head 1
    out, fs = fwd(q, k, v, la, b, cu)
    bad = np.isnan(out).any(axis=2)
    assert bad[10:16, 1].all() and not bad[:10].any() and not bad[16:].any() and not bad[:, 0].any()
    assert np.isnan(fs[1, 1]).any() and not np.isnan(fs[[0, 2]]).any() and not np.isnan(fs[1, 0]).any()


# -- P14: a retained state continues the scan (initial_state) -------------------
# The per-head state is all a sample carries forward (explainer page, "What O(N)
# buys in memory and latency"); starting from S_0 the state after the sample is the
# affine map S_L = Phi S_0 + S_L(0) with Phi the product of the transition matrices.
def pin_initial_state(fwd, seed=12):
    rng = np.random.default_rng(seed)
    lens, H, dk, dv = (9, 0, 14), 2, 5, 4
    q, k, v, la, b, cu = _rand_case(rng, lens, H, dk, dv)
    N = len(lens)
    s0 = rng.standard_normal((N, H, dk, dv))
    out, fs = fwd(q, k, v, la, b, cu, initial_state=s0)
    ob, fb = brute.scan_matrices(q, k, v, la, b, cu, initial_state=s0)
    assert _rel(out, ob) < 1e-12, _rel(out, ob)
    assert _rel(fs, fb) < 1e-12, _rel(fs, fb)
    # affine in S_0: S_L(S_0) - S_L(0) = Phi S_0; an empty sample returns S_0 itself
    _, f0 = fwd(q, k, v, la, b, cu)
    for n in range(N):
        for h in range(H):
            phi = brute.transition_product(k, la, b, cu[n], cu[n + 1], h)
            assert np.allclose(fs[n, h] - f0[n, h], phi @ s0[n, h], rtol=1e-11, atol=1e-12)
    assert np.array_equal(fs[1], s0[1])
    # zero initial state is the plain scan, bit for bit
    o2, f2 = fwd(q, k, v, la, b, cu, initial_state=np.zeros_like(s0))
    o1, f1 = fwd(q, k, v, la, b, cu)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


# -- P15: splitting a sample and carrying the state gives the one-pass result ---
def pin_split_composition(fwd, seed=13):
    rng = np.random.default_rng(seed)
    L, H, dk, dv = 37, 2, 6, 3
    q, k, v, la, b, cu = _rand_case(rng, (L,), H, dk, dv)
    out, fs = fwd(q, k, v, la, b, cu)
    for a in (1, 16, 36):
        oa, fa = fwd(q[:a], k[:a], v[:a], la[:a], b[:a], np.array([0, a], np.int32))
        ob, fb = fwd(q[a:], k[a:], v[a:], la[a:], b[a:], np.array([0, L - a], np.int32),
                     initial_state=fa)
        assert np.array_equal(np.concatenate([oa, ob]), out) and np.array_equal(fb, fs)


# -- NEXT-3: per-token L2 normalisation of q and k before the recurrence ----------
# (the paper's training setup names kernels with fused normalisation; the form
# taken is q_t / |q_t|, k_t / |k_t| per (token, head), zero vectors kept zero)
def pin_l2norm_scale_invariance(fwd, seed=14):
    """Normalised inputs do not depend on the length of q_t or k_t: scaling each
    (token, head) vector by its own positive factor leaves out and state unchanged."""
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, [7, 12, 5], H=2, dk=6, dv=5, unit_keys=False)
    T, H = q.shape[:2]
    cq = rng.uniform(0.2, 5.0, (T, H, 1))
    ck = rng.uniform(0.2, 5.0, (T, H, 1))
    o1, f1 = fwd(q, k, v, la, b, cu, qk_l2norm=True)
    o2, f2 = fwd(q * cq, k * ck, v, la, b, cu, qk_l2norm=True)
    assert _rel(o2, o1) < 1e-12 and _rel(f2, f1) < 1e-12, (_rel(o2, o1), _rel(f2, f1))
    # and the option is not a no-op on keys of non-unit length
    o3, _ = fwd(q, k, v, la, b, cu)
    assert _rel(o3, o1) > 1e-3


def pin_l2norm_recall(fwd, seed=15):
    """alpha = beta = 1 with keys along orthonormal directions but of random lengths:
    after normalisation a query along a stored direction returns the latest value
    written there, whatever the lengths of the key and the query."""
    rng = np.random.default_rng(seed)
    d = 8
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    T = d + 3
    order = list(range(d)) + [2, 5, 2]
    k = np.stack([Qm[:, s] * rng.uniform(0.3, 3.0) for s in order])[:, None, :]
    v = rng.standard_normal((T, 1, d))
    src = [0, 0, 1, 3, 2, 4, 5, 1, 0, 5, 2]
    q = np.stack([Qm[:, s] * rng.uniform(0.3, 3.0) for s in src])[:, None, :]
    la = np.zeros((T, 1, d)); b = np.ones((T, 1))
    out, _ = fwd(q, k, v, la, b, np.array([0, T], np.int32), qk_l2norm=True)
    for t in range(T):
        last = max(u for u in range(t + 1) if order[u] == src[t])
        assert np.allclose(out[t, 0], v[last, 0], rtol=0, atol=1e-12), (t, src[t], last)


def pin_l2norm_zero_vectors(fwd, seed=16):
    """A zero query reads 0; a zero key writes and erases nothing, which is the
    same step as beta_t = 0 (S_t = Diag(alpha_t) S_{t-1})."""
    rng = np.random.default_rng(seed)
    q, k, v, la, b, cu = _rand_case(rng, [9, 6], H=2, dk=4, dv=3, unit_keys=False)
    zq = [(1, 0), (4, 1), (10, 0)]
    zk = [(2, 1), (5, 0), (12, 1)]
    q0 = q.copy(); k0 = k.copy(); b0 = b.copy()
    for t, h in zq:
        q0[t, h] = 0.0
    for t, h in zk:
        k0[t, h] = 0.0
        b0[t, h] = 0.0
    out, fs = fwd(q0, k0, v, la, b, cu, qk_l2norm=True)
    ref, rfs = fwd(q0, np.where(k0 == 0.0, k, k0), v, la, b0, cu, qk_l2norm=True)
    for t, h in zq:
        assert np.all(out[t, h] == 0.0)
    assert _rel(out, ref) < 1e-13 and _rel(fs, rfs) < 1e-13


def pin_l2norm_scalar(fwd, seed=17):
    """d_k = 1: normalisation keeps only signs, s_t = alpha_t (1 - beta_t) s_{t-1} +
    beta_t sgn(k_t) v_t and o_t = sgn(q_t) s_t, solved by cumulative products."""
    rng = np.random.default_rng(seed)
    T = 30
    k = rng.uniform(-3, 3, (T, 1, 1)); v = rng.standard_normal((T, 1, 1))
    q = rng.uniform(-3, 3, (T, 1, 1)); la = -rng.uniform(0, 0.5, (T, 1, 1))
    b = rng.uniform(0, 1, (T, 1))
    out, fs = fwd(q, k, v, la, b, np.array([0, T], np.int32), qk_l2norm=True)
    a = np.exp(la[:, 0, 0]) * (1 - b[:, 0])
    c = b[:, 0] * np.sign(k[:, 0, 0]) * v[:, 0, 0]
    s = np.array([sum(np.prod(a[r + 1:t + 1]) * c[r] for r in range(t + 1)) for t in range(T)])
    assert np.allclose(out[:, 0, 0], s * np.sign(q[:, 0, 0]), rtol=1e-11, atol=1e-13)
    assert np.isclose(fs[0, 0, 0, 0], s[-1], rtol=1e-11, atol=1e-13)


ALL_PINS = [pin_worked_example, pin_brute_force, pin_beta_zero, pin_exact_recall, pin_half_life,
            pin_reset_and_packing, pin_write_readback, pin_column_separability, pin_linearity,
            pin_channel_equivariance, pin_scalar_closed_form, pin_lms_step, pin_contraction,
            pin_nan_confined, pin_initial_state, pin_split_composition,
            pin_l2norm_scale_invariance, pin_l2norm_recall, pin_l2norm_zero_vectors, pin_l2norm_scalar]
