"""Independent fp64 forms of the KDA operator -- TEST INFRASTRUCTURE ONLY.

Used to pin the C recurrence (kda_oracle.c) against forms that share none of
its code.  All functions work on one sequence and one head:

    q, k : [T, dk]   v : [T, dv]   log_alpha : [T, dk]   beta : [T]
    S0   : [dk, dv]  (state rows are key channels)

returning (o [T, dv], S_T [dk, dv]) in fp64.
"""
from __future__ import annotations

import numpy as np


def transitions(k, log_alpha, beta):
    """Per-token dk x dk transitions A_t = (I - beta_t k_t k_t^T) Diag(alpha_t).

    This is the DPLR matrix Diag(alpha) - a b^T with a = beta k and
    b = alpha (.) k ("Kimi Linear" page, "The constrained DPLR form and the
    chunkwise algorithm").
    """
    T, dk = k.shape
    A = np.empty((T, dk, dk))
    eye = np.eye(dk)
    for t in range(T):
        A[t] = (eye - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(log_alpha[t]))
    return A


def brute(q, k, v, log_alpha, beta, S0):
    """S_t = A_t S_{t-1} + beta_t k_t v_t^T with explicit dense A_t; o_t = S_t^T q_t."""
    A = transitions(k, log_alpha, beta)
    S = np.array(S0, dtype=np.float64)
    o = np.empty((len(q), v.shape[1]))
    for t in range(len(q)):
        S = A[t] @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def attention_form(q, k, v, log_alpha, beta, S0):
    """Unrolled sum: o_t = sum_i beta_i (k_i^T M_{t,i}^T q_t) v_i + (M_{t,-1} S0)^T q_t,

    where M_{t,i} = A_t A_{t-1} ... A_{i+1} is the cumulative product of
    transitions between write i and read t ("Kimi Linear" page, "Why
    channel-wise gating matters": the query dotted with keys weighted by a
    cumulative product of transition matrices).  O(T^2 dk^3): tiny T only.
    """
    A = transitions(k, log_alpha, beta)
    T, dk = k.shape
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        M = np.eye(dk)  # M_{t,t}
        for i in range(t, -1, -1):
            # M = A_t ... A_{i+1}
            o[t] += beta[i] * (k[i] @ (M.T @ q[t])) * v[i]
            M = M @ A[i]
        # M = A_t ... A_0
        o[t] += (M @ S0).T @ q[t]
    S = np.array(S0, dtype=np.float64)
    for t in range(T):
        S = A[t] @ S + beta[t] * np.outer(k[t], v[t])
    return o, S


def forward_substitution(Atil):
    """T = (I + Atil)^{-1} for strictly lower-triangular Atil, row by row.

    T_{r,:r} = -Atil_{r,:r} T_{:r,:r}, T_{rr} = 1 (the UT transform of the
    "Kimi Linear" page, "The constrained DPLR form and the chunkwise algorithm").
    """
    n = Atil.shape[0]
    T = np.eye(n)
    for r in range(1, n):
        T[r, :r] = -Atil[r, :r] @ T[:r, :r]
    return T


def chunkwise(q, k, v, log_alpha, beta, S0, C=64, solve="substitution"):
    """Chunked WY/UT evaluation of the same recurrence (derived from it).

    Within a chunk of n tokens with start state S, with G_r = sum_{j<=r} g_j
    (chunk-local inclusive cumsum of log_alpha, per key channel):

      Atil[r,i] = beta_r sum_c k_rc k_ic exp(G_rc - G_ic)   (i < r)
      Tm        = (I + Atil)^{-1}
      W         = Tm diag(beta) (K * exp(G))       Util = Tm diag(beta) V
      U         = Util - W S
      P[r,i]    = sum_c q_rc k_ic exp(G_rc - G_ic)      (i <= r)
      O         = (Q * exp(G)) S + P U
      S_next    = Diag(exp(G_last)) S + (K * exp(G_last - G))^T U

    The products use exp(G_r - G_i) formed pairwise, so nothing overflows.
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        b = beta[c0:c1]
        G = np.cumsum(log_alpha[c0:c1], axis=0)
        D = np.exp(G[:, None, :] - G[None, :, :])           # [r, i, c] = exp(G_rc - G_ic)
        kk = np.einsum("rc,ic,ric->ri", K, K, D)
        qk = np.einsum("rc,ic,ric->ri", Q, K, D)
        Atil = np.tril(b[:, None] * kk, -1)
        P = np.tril(qk)
        if solve == "substitution":
            Tm = forward_substitution(Atil)
        else:
            Tm = np.linalg.inv(np.eye(len(b)) + Atil)
        W = Tm @ (b[:, None] * (K * np.exp(G)))
        Ut = Tm @ (b[:, None] * V)
        U = Ut - W @ S
        o[c0:c1] = (Q * np.exp(G)) @ S + P @ U
        S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ U
    return o, S
