"""An independent float64 formulation used to pin the oracle.

Instead of the elementwise delta-rule update, each token applies the
generalised Householder transition that the fused_recurrent page's "M
Householder copies" refers to, written as explicit matrix products:

    A_t = a_t (I - beta_t k_t k_t^T)          (K x K)
    S_t = A_t S_{t-1} + beta_t k_t v_t^T       (K x V)
    o_t = scale * S_t^T q_t

Expanding A_t S + beta k v^T gives a S + k (beta (v - (a S)^T k))^T, the
elementwise form, so the two must agree up to float32 rounding.  A second
check unrolls the recurrence into the closed form
    S_T = (A_T ... A_1) S_0 + sum_j (A_T ... A_{j+1}) beta_j k_j v_j^T .
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2n(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.dot(x, x) + EPS)


def dense_walk(S0, qs, ks, vs, a, beta, scale, l2norm):
    """S0 [K, V]; qs, ks [T, K]; vs [T, V]; a, beta [T] (beta may be [T, V]).
    Returns (o [T, V], S_T [K, V]) in float64."""
    S = np.array(S0, dtype=np.float64)
    K = S.shape[0]
    T = len(qs)
    outs = []
    for t in range(T):
        k = l2n(ks[t]) if l2norm else np.asarray(ks[t], np.float64)
        q = l2n(qs[t]) if l2norm else np.asarray(qs[t], np.float64)
        b = np.asarray(beta[t], dtype=np.float64)
        if b.ndim == 0:
            A = float(a[t]) * (np.eye(K) - float(b) * np.outer(k, k))
            S = A @ S + float(b) * np.outer(k, np.asarray(vs[t], np.float64))
        else:
            # a per-column beta gives each V column its own transition
            cols = []
            for j in range(S.shape[1]):
                A = float(a[t]) * (np.eye(K) - b[j] * np.outer(k, k))
                cols.append(A @ S[:, j] + b[j] * k * float(vs[t][j]))
            S = np.stack(cols, axis=1)
        outs.append(scale * (S.T @ q))
    return np.array(outs).reshape(T, S.shape[1]), S


def unrolled_state(S0, ks, vs, a, beta, l2norm):
    """The closed form of the final state as products of transitions."""
    S0 = np.array(S0, dtype=np.float64)
    K = S0.shape[0]
    T = len(ks)
    kh = [l2n(ks[t]) if l2norm else np.asarray(ks[t], np.float64) for t in range(T)]
    A = [float(a[t]) * (np.eye(K) - float(beta[t]) * np.outer(kh[t], kh[t])) for t in range(T)]

    def prod(lo, hi):  # A_hi ... A_lo (latest on the left), 0-based inclusive
        P = np.eye(K)
        for s in range(lo, hi + 1):
            P = A[s] @ P
        return P

    S = prod(0, T - 1) @ S0
    for j in range(T):
        S = S + prod(j + 1, T - 1) @ (float(beta[j]) * np.outer(kh[j], np.asarray(vs[j], np.float64)))
    return S
