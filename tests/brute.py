"""Second, independent formulation of the KDA scan for tiny inputs (tests only).

Instead of the oracle's expanded token update, this builds every transition
matrix M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) as a dense d_k x d_k array
(Chimera explainer, "One stream, three mechanisms, no positions") and applies
S_t = M_t S_{t-1} + beta_t k_t v_t^T; it also evaluates the unrolled sum
S_L = sum_s (M_L ... M_{s+1}) beta_s k_s v_s^T directly.
"""
import numpy as np


def transition(k, alpha, beta):
    dk = k.shape[0]
    return (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(alpha)


def scan_matrices(q, k, v, log_alpha, beta, cu_seqlens, initial_state=None):
    """Dense-matrix recurrence. Shapes as the oracle: [T, H, d]; initial_state
    [N, H, dk, dv] or None (zero states)."""
    T, H, dk = k.shape
    dv = v.shape[2]
    N = len(cu_seqlens) - 1
    out = np.zeros((T, H, dv))
    fs = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[n, h], float)
            for t in range(cu_seqlens[n], cu_seqlens[n + 1]):
                M = transition(k[t, h], np.exp(log_alpha[t, h]), beta[t, h])
                S = M @ S + beta[t, h] * np.outer(k[t, h], v[t, h])
                out[t, h] = S.T @ q[t, h]
            fs[n, h] = S
    return out, fs


def final_state_unrolled(k, v, log_alpha, beta, t0, t1, h):
    """S at the end of tokens [t0, t1) of head h as the sum over writes."""
    dk, dv = k.shape[2], v.shape[2]
    Ms = [transition(k[t, h], np.exp(log_alpha[t, h]), beta[t, h]) for t in range(t0, t1)]
    S = np.zeros((dk, dv))
    for s in range(t0, t1):
        P = np.eye(dk)
        for t in range(s + 1, t1):
            P = Ms[t - t0] @ P
        S += P @ (beta[s, h] * np.outer(k[s, h], v[s, h]))
    return S


def transition_product(k, log_alpha, beta, t0, t1, h):
    """M_{t1-1} ... M_{t0}: the linear part of the map from the state before t0 to
    the state after t1 - 1."""
    dk = k.shape[2]
    P = np.eye(dk)
    for t in range(t0, t1):
        P = transition(k[t, h], np.exp(log_alpha[t, h]), beta[t, h]) @ P
    return P
