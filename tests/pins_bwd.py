"""Checks that pin the fp64 reverse-mode oracle (kda_oracle_backward) to facts outside it.

Each check takes ``fwd`` and ``bwd`` (oracle.forward / oracle.backward or the same
functions of another build) and raises AssertionError on a mismatch:
  - central finite differences of the forward oracle (itself pinned by pins.py) along
    random directions, one input at a time, over packed samples with an initial state
    and a final-state gradient, with and without the q/k normalisation;
  - torch float64 autograd through the dense transition-matrix form
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t
    (explainer page, "One stream, three mechanisms, no positions"), an independent
    formulation differentiated by a library.
"""
import numpy as np

NAMES = ("q", "k", "v", "log_alpha", "beta", "initial_state")


def _case(seed, lens=(7, 0, 13, 5), H=2, dk=5, dv=4, unit_keys=True):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=2, keepdims=True)
    else:
        k *= rng.uniform(0.3, 3.0, (T, H, 1))
    v = rng.standard_normal((T, H, dv))
    la = -rng.uniform(0.01, 0.3, (T, H, dk))
    b = rng.uniform(0.0, 1.0, (T, H))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = len(lens)
    s0 = rng.standard_normal((N, H, dk, dv)) * 0.5
    do = rng.standard_normal((T, H, dv))
    dfs = rng.standard_normal((N, H, dk, dv))
    return rng, [q, k, v, la, b, s0], cu, do, dfs


def _check_fd(fwd, bwd, seed, norm):
    rng, x, cu, do, dfs = _case(seed, unit_keys=not norm)
    g = bwd(*x[:5], cu, do, dfs, initial_state=x[5], qk_l2norm=norm)

    def loss(args):
        o, f = fwd(*args[:5], cu, initial_state=args[5], qk_l2norm=norm)
        return float((o * do).sum() + (f * dfs).sum())

    eps = 1e-6
    for i, name in enumerate(NAMES):
        d = rng.standard_normal(x[i].shape)
        xp = list(x); xm = list(x)
        xp[i] = x[i] + eps * d
        xm[i] = x[i] - eps * d
        fd = (loss(xp) - loss(xm)) / (2 * eps)
        an = float((g[i] * d).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, norm, fd, an)


def pin_bwd_finite_differences(fwd, bwd, seed=30):
    _check_fd(fwd, bwd, seed, norm=False)


def pin_bwd_finite_differences_normalised(fwd, bwd, seed=31):
    _check_fd(fwd, bwd, seed, norm=True)


def _dense_autograd(x, cu, do, dfs, norm):
    import torch
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in x]
    q, k, v, la, b, s0 = t
    T, H, dk = q.shape
    loss = torch.zeros((), dtype=torch.float64)
    eye = torch.eye(dk, dtype=torch.float64)
    for n in range(len(cu) - 1):
        for h in range(H):
            S = s0[n, h]
            for s in range(int(cu[n]), int(cu[n + 1])):
                kt, qt = k[s, h], q[s, h]
                if norm:
                    kt = kt / torch.linalg.vector_norm(kt)
                    qt = qt / torch.linalg.vector_norm(qt)
                M = (eye - b[s, h] * torch.outer(kt, kt)) @ torch.diag(torch.exp(la[s, h]))
                S = M @ S + b[s, h] * torch.outer(kt, v[s, h])
                loss = loss + (S.T @ qt * torch.tensor(do[s, h])).sum()
            loss = loss + (S * torch.tensor(dfs[n, h])).sum()
    loss.backward()
    return [a.grad.numpy() for a in t]


def _check_autograd(bwd, seed, norm):
    _, x, cu, do, dfs = _case(seed, lens=(6, 9, 0, 4), H=2, dk=4, dv=3, unit_keys=not norm)
    g = bwd(*x[:5], cu, do, dfs, initial_state=x[5], qk_l2norm=norm)
    ref = _dense_autograd(x, cu, do, dfs, norm)
    for name, a, r in zip(NAMES, g, ref):
        assert np.allclose(a, r, rtol=1e-10, atol=1e-12), (name, norm, np.abs(a - r).max())


def pin_bwd_dense_autograd(fwd, bwd, seed=32):
    _check_autograd(bwd, seed, norm=False)


def pin_bwd_dense_autograd_normalised(fwd, bwd, seed=33):
    _check_autograd(bwd, seed, norm=True)


def pin_bwd_no_initial_state(fwd, bwd, seed=34):
    """Without an initial state the gradients are those of the run from zero states,
    and d_initial_state is still the gradient with respect to those zeros."""
    _, x, cu, do, dfs = _case(seed)
    zero = np.zeros_like(x[5])
    g0 = bwd(*x[:5], cu, do, dfs)
    g1 = bwd(*x[:5], cu, do, dfs, initial_state=zero)
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)
    ref = _dense_autograd(x[:5] + [zero], cu, do, dfs, False)
    assert np.allclose(g0[5], ref[5], rtol=1e-10, atol=1e-12)


ALL_BWD_PINS = [pin_bwd_finite_differences, pin_bwd_finite_differences_normalised,
                pin_bwd_dense_autograd, pin_bwd_dense_autograd_normalised, pin_bwd_no_initial_state]
